// Internal declarations shared by the host validation code and the HIP
// launch code of the verify-attention library (not part of the C ABI).
#ifndef MLA_VERIFY_INTERNAL_H
#define MLA_VERIFY_INTERNAL_H

#include <cstddef>
#include <initializer_list>

#include "mla_verify.h"

namespace mla {

constexpr int kNumCUs = 256;           // MI355X compute units
constexpr int kNumXCDs = 8;            // dies; workgroups are dealt to them round-robin
constexpr size_t kL2BytesPerXCD = 4u << 20;   // each die's L2
constexpr int kMaxSplitPages = 1024;   // block-table entries one split stages in LDS
constexpr int kMaxBalancedBatch = 2000;   // requests whose unit prefix sums fit the kernel's LDS

// Shape of one attention workgroup (always four wavefronts).
//   mode 0: 32-row tile, 64-key staging units, QK split by keys
//   mode 1: 64-row tile, 64-key staging units, QK split by keys
// In modes 0 and 1 PV splits the 512 latent dims between the four waves.
//   mode 3: 128-row tile, 32-key staging units (attn_rows_kernel, bf16 or fp8
//           cache): each wave owns 32 rows for QK, softmax and PV alike
struct TileShape {
  int mode;
  int tile_rows() const { return mode == 0 ? 32 : (mode == 1 ? 64 : 128); }
};

struct Plan {
  int rows;             // R = T * H folded rows per request
  TileShape shape;
  int row_tiles;        // ceil(R / tile rows)
  int splits;           // S
  int min_split_pages;  // m: a request of n pages takes min(S, ceil(n / m)) splits
  bool use_partials;    // results go through the partial workspace (bf16 O, fp32 LSE)
  bool balanced;        // mode 3 with S >= 2: balanced chunks instead of per-tile splits
  int chunk_min;        // balanced chunks: minimum chunk in 32-key units, ceil(2 P / (S - 1))
  size_t workspace_bytes;
};

TileShape choose_shape(int rows, int batch, int forced_splits);
int check_params(const mla_verify_params* p);
Plan make_plan(const mla_verify_params* p, bool gated);
bool aligned16(const void* ptr);
bool any_null(std::initializer_list<const void*> ptrs);
bool any_misaligned(std::initializer_list<const void*> ptrs);   // any non-null pointer not 16-byte aligned
// Device set-up check (gfx950, kernel attributes); defined with the
// attention kernels.
int device_ready();
// Sizes of the KV append / trim calls (pure host checks).
int check_kv_dims(int batch, int q_len, int max_pages_per_req, int num_pool_pages);

}  // namespace mla

#endif
