// Internal declarations shared by the host validation code and the HIP
// launch code of the verify-attention library (not part of the C ABI).
#ifndef MLA_VERIFY_INTERNAL_H
#define MLA_VERIFY_INTERNAL_H

#include <cstddef>

#include "mla_verify.h"

namespace mla {

constexpr int kTileRows = 32;   // folded rows per attention workgroup
constexpr int kNumCUs = 256;    // MI355X compute units
constexpr int kNumXCDs = 8;     // dies; workgroups are dealt to them round-robin
constexpr int kMaxSplitPages = 1024;   // block-table entries one split stages in LDS

struct Plan {
  int rows;             // R = T * H folded rows per request
  int row_tiles;        // ceil(R / kTileRows)
  int splits;           // S
  bool use_partials;    // results go through the fp32 partial workspace
  size_t workspace_bytes;
};

int check_params(const mla_verify_params* p);
Plan make_plan(const mla_verify_params* p, bool gated);
bool aligned16(const void* ptr);

}  // namespace mla

#endif
