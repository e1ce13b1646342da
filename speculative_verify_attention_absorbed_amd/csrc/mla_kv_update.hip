// HIP kernels and C-ABI entry points of the paged-cache updates around a
// verify step (gfx950): the group's latents appended by a per-token slot
// table, and the trim of rejected tails after verification.  See
// include/mla_verify.h for the passages followed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_launch.h"
#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace {

constexpr int D = MLA_VERIFY_LATENT;   // 512
constexpr int PG = MLA_VERIFY_PAGE;    // 64
constexpr int kThreads = 256;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// KV append with a per-token slot table: one wave per token of a group; its
// 1 KiB latent row goes to the page and slot its table entry names (-1:
// another rank owns the token, nothing to write).  Out-of-range slots and
// page ids write nothing and are counted.
__global__ __launch_bounds__(kThreads) void kv_append_kernel(const uint16_t* __restrict__ new_latent,
                                                             const int32_t* __restrict__ slots,
                                                             const int32_t* __restrict__ bt,
                                                             uint16_t* __restrict__ pool,
                                                             int32_t* __restrict__ bad, int tokens, int T,
                                                             int P, int N) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= tokens) return;
  const int lane = threadIdx.x & 63;
  const int b = tok / T;
  const int slot = __builtin_amdgcn_readfirstlane(slots[tok]);
  if (slot == -1) return;
  const bool in_row = slot >= 0 && slot < P * PG;
  const int pid = in_row ? __builtin_amdgcn_readfirstlane(bt[(size_t)b * P + slot / PG]) : -1;
  if (!in_row || pid < 0 || pid >= N) {
    if (lane == 0 && bad != nullptr) atomicAdd(bad, 1);
    return;
  }
  const uint4 v = *reinterpret_cast<const uint4*>(new_latent + (size_t)tok * D + lane * 8);
  *reinterpret_cast<uint4*>(pool + ((size_t)pid * PG + (slot & (PG - 1))) * D + lane * 8) = v;
}

// Trim of rejected tails: one thread per request.  The dropped keys are the
// last T - 1 - accepted (< 16 < 64) of the request, so at most one page holds
// nothing but dropped keys; it is released from the block table.
__global__ __launch_bounds__(kThreads) void kv_trim_kernel(const int32_t* kv_len, const int32_t* accepted,
                                                           int32_t* new_len, int32_t* bt, int32_t* released,
                                                           int B, int T, int P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= B) return;
  const int L = clampi(kv_len[b], 0, P * PG);
  const int a = clampi(accepted[b], 0, T - 1);
  const int nl = max(0, L - (T - 1 - a));
  const int p_lo = (nl + PG - 1) / PG, p_hi = (L + PG - 1) / PG;
  int rel = -1;
  if (p_lo < p_hi) {
    int32_t* e = bt + (size_t)b * P + p_lo;
    rel = *e;
    *e = -1;
  }
  new_len[b] = nl;
  released[b] = rel;
}

}  // namespace

extern "C" {

int mla_verify_kv_append(int batch, int q_len, int max_pages_per_req, int num_pool_pages,
                         const mla_bf16* new_latent, const int32_t* slots, const int32_t* block_table,
                         mla_bf16* latent_kv_pages, int32_t* bad_slots, void* stream) {
  int rc = mla::check_kv_dims(batch, q_len, max_pages_per_req, num_pool_pages);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({new_latent, slots, block_table, latent_kv_pages})) return MLA_ERR_NULL;
  if (mla::any_misaligned({new_latent, slots, block_table, latent_kv_pages})) return MLA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(bad_slots) & 3u) != 0) return MLA_ERR_ARG;
  rc = mla::device_ready();
  if (rc != MLA_OK) return rc;
  const int tokens = batch * q_len;
  return mla::launch(kv_append_kernel, dim3((tokens + 3) / 4), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     new_latent, slots, block_table, latent_kv_pages, bad_slots, tokens, q_len, max_pages_per_req,
                     num_pool_pages);
}

int mla_verify_kv_trim(int batch, int q_len, int max_pages_per_req, const int32_t* kv_len,
                       const int32_t* accepted, int32_t* new_len, int32_t* block_table,
                       int32_t* released_page, void* stream) {
  int rc = mla::check_kv_dims(batch, q_len, max_pages_per_req, 1);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({kv_len, accepted, new_len, block_table, released_page})) return MLA_ERR_NULL;
  if (mla::any_misaligned({kv_len, accepted, new_len, block_table, released_page})) return MLA_ERR_ARG;
  rc = mla::device_ready();
  if (rc != MLA_OK) return rc;
  return mla::launch(kv_trim_kernel, dim3((batch + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), kv_len, accepted, new_len, block_table, released_page, batch,
                     q_len, max_pages_per_req);
}

}  // extern "C"
