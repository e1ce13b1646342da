// Host-side argument validation and planning for the verify-attention C ABI.
// Pure C++: nothing here touches the HIP runtime, so every error path can be
// exercised on a machine without a GPU.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace mla {

int check_params(const mla_verify_params* p) {
  if (p == nullptr) return MLA_ERR_NULL;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3) return MLA_ERR_DTYPE;
  if (p->kv_dtype == MLA_KV_FP8_E4M3 && (!std::isfinite(p->kv_scale) || !(p->kv_scale > 0.0f)))
    return MLA_ERR_ARG;
  if (p->latent_dim != MLA_VERIFY_LATENT || p->page_size != MLA_VERIFY_PAGE) return MLA_ERR_SHAPE;
  if (p->batch < 1 || p->q_len < 1 || p->q_len > MLA_VERIFY_MAX_Q_LEN || p->num_heads < 1 ||
      p->num_heads > MLA_VERIFY_MAX_HEADS)
    return MLA_ERR_SHAPE;
  if (p->max_pages_per_req < 1 || p->num_pool_pages < 1) return MLA_ERR_ARG;
  // keep every index computation comfortably inside int32 / size_t
  if ((int64_t)p->max_pages_per_req * MLA_VERIFY_PAGE > (int64_t)1 << 30) return MLA_ERR_ARG;
  if ((int64_t)p->batch * p->max_pages_per_req > (int64_t)1 << 30) return MLA_ERR_ARG;
  if ((int64_t)p->batch * p->q_len * p->num_heads > (int64_t)1 << 24) return MLA_ERR_SHAPE;
  if (p->num_splits < 0 || p->num_splits > MLA_VERIFY_MAX_SPLITS) return MLA_ERR_ARG;
  if (p->tile_rows != 0 && p->tile_rows != 32 && p->tile_rows != 64 && p->tile_rows != 128)
    return MLA_ERR_ARG;
  if (!std::isfinite(p->sm_scale) || !(p->sm_scale > 0.0f)) return MLA_ERR_ARG;
  // a forced split count must keep every split within kMaxSplitPages pages
  if (p->num_splits > 0 &&
      (p->max_pages_per_req + p->num_splits - 1) / p->num_splits > kMaxSplitPages)
    return MLA_ERR_ARG;
  if ((p->max_pages_per_req + kMaxSplitPages - 1) / kMaxSplitPages > MLA_VERIFY_MAX_SPLITS)
    return MLA_ERR_ARG;
  return MLA_OK;
}

// Library's choice of tile (when tile_rows == 0).  Up to 32 folded rows: one
// 32-row tile.  Up to 64: one 64-row tile stages each page once per split,
// while two 32-row tiles stage it twice (the second read hits L2) but need
// half the splits to fill the GPU, so every row has half as many partials to
// write and merge.  A tile's staging and LDS traffic per page do not depend
// on how many of its rows are real, so the second 32-row tile is worth it
// only when it is more than half full (more than 48 rows) and the pair still
// leaves at least four splits per tile at one workgroup per CU (few, long
// requests); otherwise the 64-row tile.  With a forced split count the
// tiles are chosen to fill the GPU instead: two 32-row tiles while that still
// fits one workgroup per CU, else one 64-row tile.  More rows: 128-row tiles
// (each wave owns 32 rows in QK), which keep the number of times a page is
// re-staged small.
TileShape choose_shape(int rows, int batch, int forced_splits) {
  if (rows <= 32) return TileShape{0};
  if (rows <= 64) {
    if (forced_splits > 0)
      return (int64_t)batch * forced_splits * 2 <= kNumCUs ? TileShape{0} : TileShape{1};
    return rows > 48 && (int64_t)kNumCUs / ((int64_t)batch * 2) >= 4 ? TileShape{0} : TileShape{1};
  }
  return TileShape{3};
}

TileShape shape_for_rows(int tile_rows) {
  return TileShape{tile_rows == 32 ? 0 : (tile_rows == 64 ? 1 : 3)};
}

Plan make_plan(const mla_verify_params* p, bool gated) {
  Plan pl{};
  pl.rows = p->q_len * p->num_heads;
  pl.shape = p->tile_rows != 0 ? shape_for_rows(p->tile_rows)
                               : choose_shape(pl.rows, p->batch, p->num_splits);
  pl.row_tiles = (pl.rows + pl.shape.tile_rows() - 1) / pl.shape.tile_rows();
  int s = p->num_splits;
  if (s == 0) {
    // Library's choice: enough workgroups to give every CU one (a workgroup
    // holds ~150 KiB of LDS, so one fits per CU; a second round of
    // workgroups costs more than it saves), and at least one split per 16
    // pages of the longest possible request, so that a long request in a
    // ragged batch is not left to a single workgroup (shorter requests then
    // take fewer splits, see min_split_pages); never more splits than pages.
    const int64_t tiles = (int64_t)p->batch * pl.row_tiles;
    int64_t want = kNumCUs / tiles;
    const int64_t by_len = (p->max_pages_per_req + 15) / 16;
    if (want < by_len) want = by_len;
    if (want > p->max_pages_per_req) want = p->max_pages_per_req;
    if (want > MLA_VERIFY_MAX_SPLITS) want = MLA_VERIFY_MAX_SPLITS;
    s = want < 1 ? 1 : (int)want;
  }
  // one split stages at most kMaxSplitPages block-table entries
  const int min_s = (p->max_pages_per_req + kMaxSplitPages - 1) / kMaxSplitPages;
  if (p->num_splits == 0 && s < min_s) s = min_s;
  pl.splits = s;
  // Splits adapt to each request's own length: at least half the pages the
  // longest possible request puts in one split.  For a batch of similar
  // lengths this gives S splits per request; in a ragged one a short request
  // takes fewer (each split is a workgroup with a fixed setup cost).
  const int per_split = (p->max_pages_per_req + s - 1) / s;
  pl.min_split_pages = per_split / 2 > 1 ? per_split / 2 : 1;
  pl.use_partials = gated || s > 1;
  // 128-row tiles with a split count: balanced chunks.  A request of at
  // most 2 P units spans at most floor((2P - 1) / C) + 2 chunks, which is <= S
  // once C >= ceil(2P / (S - 1)).  A chunk can hold more pages of one request
  // than a workgroup stages block-table entries, so balanced chunks need the
  // whole block-table row to fit (P <= kMaxSplitPages); longer rows take the
  // per-tile splits, whose page count per split the argument check bounds.
  pl.balanced = pl.shape.mode == 3 && s >= 2 && p->batch <= kMaxBalancedBatch &&
                p->max_pages_per_req <= kMaxSplitPages;
  pl.chunk_min = pl.balanced ? (2 * p->max_pages_per_req + s - 2) / (s - 1) : 0;
  const size_t total_rows = (size_t)p->batch * pl.rows;
  // partial outputs in bf16, partial LSEs in fp32
  pl.workspace_bytes =
      pl.use_partials ? (size_t)s * total_rows * (MLA_VERIFY_LATENT * 2 + sizeof(float)) : 0;
  return pl;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool any_null(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x == nullptr) return true;
  return false;
}

bool any_misaligned(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x != nullptr && !aligned16(x)) return true;
  return false;
}

int check_kv_dims(int batch, int q_len, int max_pages_per_req, int num_pool_pages) {
  if (batch < 1 || q_len < 1 || q_len > MLA_VERIFY_MAX_Q_LEN) return MLA_ERR_SHAPE;
  if (max_pages_per_req < 1 || num_pool_pages < 1) return MLA_ERR_ARG;
  // slot and table indices stay inside int32
  if ((int64_t)max_pages_per_req * MLA_VERIFY_PAGE > (int64_t)1 << 30) return MLA_ERR_ARG;
  if ((int64_t)batch * max_pages_per_req > (int64_t)1 << 30) return MLA_ERR_ARG;
  if ((int64_t)batch * q_len > (int64_t)1 << 24) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace mla

extern "C" {

int mla_verify_check(const mla_verify_params* p) { return mla::check_params(p); }

int mla_verify_tile_rows(const mla_verify_params* p, int gated) {
  const int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  return mla::make_plan(p, gated != 0).shape.tile_rows();
}

int mla_verify_num_splits(const mla_verify_params* p, int gated) {
  const int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  return mla::make_plan(p, gated != 0).splits;
}

int mla_verify_workspace_size(const mla_verify_params* p, int gated, size_t* bytes) {
  if (bytes == nullptr) return MLA_ERR_NULL;
  const int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  *bytes = mla::make_plan(p, gated != 0).workspace_bytes;
  return MLA_OK;
}

const char* mla_verify_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "unsupported shape (latent must be 512, page 64, 1<=T<=16, 1<=H<=128)";
    case MLA_ERR_DTYPE: return "unsupported KV dtype (attention takes bf16 or fp8 E4M3 latent pages; cache updates take bf16)";
    case MLA_ERR_ARG: return "invalid argument (sm_scale, num_splits, pool/page counts or alignment)";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small (allocation-free call: needs more than its static scratch)";
    case MLA_ERR_DEVICE: return "no GPU visible, or the current device is not gfx950 (MI355X)";
    case MLA_ERR_HIP: return "HIP runtime or kernel launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
