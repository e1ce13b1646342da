// HIP kernels (gfx950 / CDNA4) and C-ABI entry points of the speculative-verify
// attention library for gated NoPE MLA with absorbed projections.
//
// Method (see include/mla_verify.h for the passages followed): every request
// brings T = k+1 query tokens; tokens are folded into the head dimension
// (row r = t*H + h, token r / H), so one request is one "decode row" of
// R = T*H folded rows that streams the paged 512-d latent cache once.  Each
// folded row has its own bound kv_bounds[b, r / H].
//
// Kernels:
//   verify_attn_kernel   one workgroup per (request, 64-row tile, KV split).
//                        4 waves x 16 rows.  Per 64-key page: the page is
//                        staged HBM -> registers -> LDS (XOR-swizzled 16-byte
//                        chunks); S^T = K Q^T on bf16 MFMA 16x16x32 with Q held
//                        in registers; masked online softmax in fp32 (exp2
//                        domain); O^T += V^T P^T on MFMA, where P^T stays in the
//                        registers the S^T accumulators produced and V^T comes
//                        from LDS through ds_read_tr16_b64 transposing reads.
//                        Writes bf16 o_lat + lse directly (one split), or
//                        normalised fp32 partials + partial lse (split-KV).
//   combine_kernel       LSE merge of the S partials of every row (rows with
//                        no visible key in any split give (-inf, 0)).
//   gated_epilogue_kernel  per head: LSE merge, then W_UV (512 -> 128) on
//                        MFMA and the sigmoid gate; optional o_lat output.
//   absorb_q_kernel      q_latent = W_UK[h]^T q_nope, fp32 accumulate, bf16.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mla_verify.h"
#include "mla_verify_internal.h"

namespace {

constexpr int D = MLA_VERIFY_LATENT;   // 512
constexpr int PG = MLA_VERIFY_PAGE;    // 64
constexpr int DV = MLA_VERIFY_NOPE;    // 128
constexpr int kThreads = 256;          // 4 waves of 64
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Position of 16-byte chunk c (0..63) of key row `key` inside the LDS page tile.
// XOR of the low four chunk bits with the key's low four bits spreads the 16
// keys a wave reads together over 16 distinct chunk slots (bank-conflict free
// for both the row reads of QK^T and the transposing reads of PV).
__device__ __forceinline__ int swz(int key, int c) { return key * 64 + (c ^ (key & 15)); }

struct AttnArgs {
  const uint16_t* q;       // [B, R, 512]
  const uint16_t* pool;    // [N, 64, 512]
  const int32_t* bt;       // [B, P]
  const int32_t* bounds;   // [B, T]
  uint16_t* out_lat;       // [B, R, 512] (direct mode)
  float* lse;              // [B, R]      (direct mode)
  float* part_o;           // [S, B*R, 512] (split mode)
  float* part_lse;         // [S, B*R]
  int B, T, H, R, P, N, S, row_tiles;
  float scale_log2;        // sm_scale * log2(e)
  int direct;              // 1: write out_lat/lse, 0: write partials
};

constexpr int kRows = mla::kTileRows;          // 32 folded rows per workgroup
// A key row of the LDS page tile is 1024 bytes of latent plus 32 bytes of
// padding: the four key rows one transposing read touches then fall on four
// disjoint 8-bank groups, and every access is one base register plus an
// immediate offset.
constexpr int kRowChunks = D / 8 + 2;          // 66 16-byte chunks per key row
constexpr int kPageChunks = PG * kRowChunks;   // 4224 chunks (67584 bytes) per page
constexpr int kPStride = PG + 8;               // bf16 per P row (padded: fewer bank conflicts)
constexpr int kMaxSplitPages = mla::kMaxSplitPages;

struct AttnSmem {
  uint4 page[2][kPageChunks];          // double-buffered latent page (padded key rows)
  uint16_t p[2][kRows * kPStride];     // P (bf16), [row][key]
  float wmax[2][4][kRows];             // per-wave row maxima of the page
  float lsum[2][4][kRows];             // per-wave denominators: [0] bf16-rounded P, [1] exact
  int32_t pages[kMaxSplitPages];       // this split's block-table slice
};

// Logical work item of a workgroup.  Hardware deals workgroups to the 8 XCDs
// round-robin (bid % 8); logical items are laid out in contiguous runs per
// XCD, so the row tiles that read the same pages share one L2.  Returns -1
// for the padding workgroups of a grid rounded up to a multiple of 8.
__device__ __forceinline__ int logical_item(int bid, int n_items) {
  const int per = (n_items + mla::kNumXCDs - 1) / mla::kNumXCDs;
  const int li = (bid % mla::kNumXCDs) * per + bid / mla::kNumXCDs;
  return li < n_items ? li : -1;
}

typedef uint4 KStage[16];

// Workgroup = 4 waves over one (request b, KV split s, 32-row tile).
//  QK^T: wave w owns keys 16w..16w+15 of every page and all 32 rows; its K
//        operand is loaded straight from HBM into registers (the MFMA A
//        layout is the cache's own row-major layout), Q^T (32 rows) stays in
//        registers.  Two register stages keep two pages in flight.  The same
//        registers are written to LDS once, where the page serves as V.
//  softmax: per-wave row maxima are exchanged through LDS; every wave then
//        derives the same running max, so rescale factors agree across waves.
//  PV:   wave w owns latent dims 128w..128w+127 for all 32 rows; V^T comes
//        from LDS through ds_read_tr16_b64, P^T through a small LDS buffer.
__global__ __launch_bounds__(kThreads) void verify_attn_kernel(AttnArgs a) {
  extern __shared__ uint4 smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int i16 = lane & 15;

  int id = logical_item(blockIdx.x, a.B * a.S * a.row_tiles);
  if (id < 0) return;
  const int rt = id % a.row_tiles;
  id /= a.row_tiles;
  const int s = id % a.S;
  const int b = id / a.S;

  const int row0 = rt * kRows;
  const int rows_here = min(kRows, a.R - row0);
  const int max_keys = a.P * PG;

  // ---- independent loads first: row bounds, tile bounds, Q
  int L[2];
  bool rvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = row0 + nt * 16 + i16;
    rvalid[nt] = r < a.R;
    L[nt] = rvalid[nt] ? clampi(a.bounds[b * a.T + r / a.H], 0, max_keys) : 0;
  }
  bf16x8 qreg[2][16];   // Q^T operand: qreg[nt][ks] = q[row r_nt][ks*32 + 8g .. +7]
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = rvalid[nt] ? row0 + nt * 16 + i16 : 0;
    const uint4* qrow = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.R + r) * D);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qreg[nt][ks] = __builtin_bit_cast(bf16x8, qrow[ks * 4 + g]);
  }
  int n_tile = 0;   // keys the tile scans: the largest bound among its tokens
  {
    const int t_lo = row0 / a.H;
    const int t_hi = (row0 + rows_here - 1) / a.H;
    for (int t = t_lo; t <= t_hi; ++t) n_tile = max(n_tile, clampi(a.bounds[b * a.T + t], 0, max_keys));
  }
  const int n_pg = (n_tile + PG - 1) / PG;
  const int p_begin = (s * n_pg) / a.S;
  const int n_my = ((s + 1) * n_pg) / a.S - p_begin;   // <= ceil(P / S) <= kMaxSplitPages

  // ---- stage this split's page ids in LDS
  for (int i = tid; i < n_my; i += kThreads) sm.pages[i] = a.bt[b * a.P + p_begin + i];
  __syncthreads();

  const int my_key = 16 * w + i16;
  // K operand of page j (0-based within the split): kst[ks] = key my_key,
  // dims ks*32 + 8g .. +7.  Slots past n_tile and bad page ids read as zero.
  auto load_page = [&](KStage& kst, int j) {
    const int pid = sm.pages[j];
    const bool ok = (unsigned)pid < (unsigned)a.N && ((p_begin + j) * PG + my_key) < n_tile;
    const uint4* src = reinterpret_cast<const uint4*>(a.pool + ((size_t)(ok ? pid : 0) * PG + my_key) * D);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const uint4 v = src[ks * 4 + g];
      kst[ks] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };

  f32x4 o[8][2];   // O^T: o[dt][nt][i] = O[row r_nt][dim 128w + 16dt + 4g + i]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};   // running row max (log2 domain), same in every wave
  // this lane's share of the denominator: lround sums the bf16-rounded P that
  // feeds PV (so the output weights sum to one), lexact the fp32 values (LSE)
  float lround[2] = {0.f, 0.f};
  float lexact[2] = {0.f, 0.f};

  KStage kA, kB;
  if (n_my > 0) load_page(kA, 0);
  if (n_my > 1) load_page(kB, 1);

  auto process = [&](KStage& kst, int j) {
    const int buf = j & 1;
    const int p = p_begin + j;
    // ---- S^T = K Q^T: sacc[nt][i] = score(key 16w + 4g + i, row r_nt)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 kv = __builtin_bit_cast(bf16x8, kst[ks]);
      sacc[0] = mfma16(kv, qreg[0][ks], sacc[0]);
      sacc[1] = mfma16(kv, qreg[1][ks], sacc[1]);
    }
    // ---- the page's keys go to LDS, where they serve as V; then the stage
    // is refilled with page j+2
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) sm.page[buf][my_key * kRowChunks + ks * 4 + g] = kst[ks];

    // ---- mask + per-wave row maxima
    const int kpos0 = p * PG + 16 * w + 4 * g;
    float sv[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (kpos0 + i) < L[nt] ? sacc[nt][i] * a.scale_log2 : -INFINITY;
        sv[nt][i] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) sm.wmax[buf][w][nt * 16 + i16] = mx;
    }
    __syncthreads();   // (A) maxima and the V page are visible

    float alpha[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = nt * 16 + i16;
      const float pm = fmaxf(fmaxf(sm.wmax[buf][0][r], sm.wmax[buf][1][r]),
                             fmaxf(sm.wmax[buf][2][r], sm.wmax[buf][3][r]));
      const float m_new = fmaxf(m[nt], pm);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;   // nothing visible yet: p = 0
      alpha[nt] = exp2f(m[nt] - m_ref);
      m[nt] = m_new;
      uint32_t pb[4];
      float ps = 0.f, pe = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = exp2f(sv[nt][i] - m_ref);
        pb[i] = bf16_rne(pv);
        ps += bf16_to_f32(pb[i]);
        pe += pv;
      }
      lround[nt] = lround[nt] * alpha[nt] + ps;
      lexact[nt] = lexact[nt] * alpha[nt] + pe;
      uint2 pw;
      pw.x = pb[0] | (pb[1] << 16);
      pw.y = pb[2] | (pb[3] << 16);
      *reinterpret_cast<uint2*>(&sm.p[buf][r * kPStride + 16 * w + 4 * g]) = pw;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      o[dt][0] *= alpha[0];
      o[dt][1] *= alpha[1];
    }
    __syncthreads();   // (B) P is visible

    // ---- O^T += V^T P^T over the page's 64 keys.  k-slots of step kk are
    // keys 32kk + 8g + (0..7) for both operands.
    const lds_s16x4* vpage = (const lds_s16x4*)(&sm.page[buf][0]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 pop[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        pop[nt] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&sm.p[buf][(nt * 16 + i16) * kPStride + 32 * kk + 8 * g]));
      // transposing read: lanes 4r..4r+3 of a 16-lane group address key row
      // kb + r (4 dims each); lane j receives dim j of those 4 rows.
      // (in 8-byte units: a key row is 2*kRowChunks units, 4 dims per unit)
      const int kb = 32 * kk + 8 * g + (i16 >> 2);
      const lds_s16x4* vrow = vpage + kb * (2 * kRowChunks) + 32 * w + (i16 & 3);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            const_cast<lds_s16x4*>(vrow + 4 * dt));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            const_cast<lds_s16x4*>(vrow + 4 * (2 * kRowChunks) + 4 * dt));
        uint4 av;
        av.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        av.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        av.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        av.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        const bf16x8 vop = __builtin_bit_cast(bf16x8, av);
        o[dt][0] = mfma16(vop, pop[0], o[dt][0]);
        o[dt][1] = mfma16(vop, pop[1], o[dt][1]);
      }
    }
    if (j + 2 < n_my) load_page(kst, j + 2);   // refill this stage with page j+2
  };

  for (int j = 0; j < n_my; j += 2) {
    process(kA, j);
    if (j + 1 < n_my) process(kB, j + 1);
  }

  // ---- denominators: lanes of a row (4 groups) then the 4 waves
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float lr = lround[nt], le = lexact[nt];
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
    le += __shfl_xor(le, 16);
    le += __shfl_xor(le, 32);
    if (g == 0) {
      sm.lsum[0][w][nt * 16 + i16] = lr;
      sm.lsum[1][w][nt * 16 + i16] = le;
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (!rvalid[nt]) continue;
    const int r = nt * 16 + i16;
    const float lr = sm.lsum[0][0][r] + sm.lsum[0][1][r] + sm.lsum[0][2][r] + sm.lsum[0][3][r];
    const float le = sm.lsum[1][0][r] + sm.lsum[1][1][r] + sm.lsum[1][2][r] + sm.lsum[1][3][r];
    const bool empty = !(lr > 0.f);   // the row max contributes P = 1 whenever a key is visible
    const float inv = empty ? 0.f : 1.f / lr;
    const float lse_val = empty ? -INFINITY : (m[nt] + log2f(le)) * kLn2;
    const size_t row_g = (size_t)b * a.R + row0 + r;
    if (a.direct) {
      uint16_t* dst = a.out_lat + row_g * D + 128 * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 wv;
        wv.x = bf16_rne(o[dt][nt][0] * inv) | (bf16_rne(o[dt][nt][1] * inv) << 16);
        wv.y = bf16_rne(o[dt][nt][2] * inv) | (bf16_rne(o[dt][nt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = wv;
      }
      if (w == 0 && g == 0) a.lse[row_g] = lse_val;
    } else {
      const size_t prow = (size_t)s * a.B * a.R + row_g;
      if (w == 0 && g == 0) a.part_lse[prow] = lse_val;
      if (empty) continue;   // the merge never reads partials with lse = -inf
      float* dst = a.part_o + prow * D + 128 * w + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[dt][nt] * inv;
    }
  }
}

// LSE merge of the S partials of one row, computed by one wave (lane owns
// dims 8*lane .. 8*lane+7).  The split LSEs are read in one round (lane s
// holds split s), then the non-empty partials are fetched eight at a time
// with all loads in flight together.  Partials of empty splits are never
// read (their workspace bytes may be stale).  Returns the row's lse.
__device__ __forceinline__ float merge_row(const float* __restrict__ part_o,
                                           const float* __restrict__ part_lse, int S,
                                           size_t stride_rows, size_t row, int lane, float out[8]) {
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  float mx = -INFINITY, wl = 0.f, total = 0.f;
  for (int s0 = 0; s0 < S; s0 += 64) {   // S <= 64: one pass in practice
    const float l = (s0 + lane < S) ? part_lse[(size_t)(s0 + lane) * stride_rows + row] : -INFINITY;
    mx = fmaxf(mx, l);
  }
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (mx == -INFINITY) {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = 0.f;
    return -INFINITY;
  }
  {
    const float l = (lane < S) ? part_lse[(size_t)lane * stride_rows + row] : -INFINITY;
    wl = (l == -INFINITY) ? 0.f : expf(l - mx);   // this lane's split weight
    total = wl;
    for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  }
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 v[8][2];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sj = s0 + j;
      ws[j] = __shfl(wl, sj < S ? sj : 0);
      ws[j] = sj < S ? ws[j] : 0.f;
      if (ws[j] > 0.f) {   // wave-uniform
        const f32x4* src = reinterpret_cast<const f32x4*>(part_o + ((size_t)sj * stride_rows + row) * D + lane * 8);
        v[j][0] = src[0];
        v[j][1] = src[1];
      } else {
        v[j][0] = v[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += ws[j] * v[j][0][e];
        acc[4 + e] += ws[j] * v[j][1][e];
      }
    }
  }
  const float inv = 1.f / total;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = acc[j] * inv;
  return mx + logf(total);
}

__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           uint16_t* __restrict__ out_lat,
                                                           float* __restrict__ lse, int rows, int S) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float v[8];
  const float l = merge_row(part_o, part_lse, S, (size_t)rows, (size_t)row, lane, v);
  uint4 w;
  w.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
  w.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
  w.z = bf16_rne(v[4]) | (bf16_rne(v[5]) << 16);
  w.w = bf16_rne(v[6]) | (bf16_rne(v[7]) << 16);
  *reinterpret_cast<uint4*>(out_lat + (size_t)row * D + lane * 8) = w;
  if (lane == 0) lse[row] = l;
}

// One workgroup per (head h, tile of 64 (b, t) rows).  Phase 1: each wave
// merges 16 rows' partials and leaves o_lat (bf16) in LDS.  Phase 2: each
// wave computes out[16 rows][128] = o_lat[16][512] . W_UV[h]^T on MFMA and
// applies sigmoid(gate).
__global__ __launch_bounds__(kThreads) void gated_epilogue_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const uint16_t* __restrict__ w_uv, const uint16_t* __restrict__ gate,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ out_lat,
    int BT, int H, int S) {
  extern __shared__ uint4 lds4[];   // 64 rows x 64 chunks (bf16 o_lat) = 64 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.x % H;
  const int tile = blockIdx.x / H;
  const int rr0 = tile * 64;
  const size_t rows = (size_t)BT * H;

  for (int r = 0; r < 16; ++r) {
    const int lr = wave * 16 + r;
    const int rr = rr0 + lr;           // (b, t) row index = b*T + t
    uint4 w = make_uint4(0, 0, 0, 0);
    if (rr < BT) {
      const size_t row = (size_t)rr * H + h;
      float v[8];
      const float l = merge_row(part_o, part_lse, S, rows, row, lane, v);
      w.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
      w.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
      w.z = bf16_rne(v[4]) | (bf16_rne(v[5]) << 16);
      w.w = bf16_rne(v[6]) | (bf16_rne(v[7]) << 16);
      if (out_lat) *reinterpret_cast<uint4*>(out_lat + row * D + lane * 8) = w;
      if (lane == 0) lse[row] = l;
    }
    lds4[swz(lr, lane)] = w;
  }
  __syncthreads();

  // out^T[d][row] would need W as A; instead C[row][d] = A[row][c] B[c][d]
  const int lr = wave * 16 + i16;      // A row owned by this lane
  f32x4 acc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wh = w_uv + (size_t)h * DV * D;
#pragma unroll 4
  for (int ks = 0; ks < 16; ++ks) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, lds4[swz(lr, ks * 4 + g)]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int d = nt * 16 + i16;
      const uint4 bv = *reinterpret_cast<const uint4*>(wh + (size_t)d * D + ks * 32 + 8 * g);
      acc[nt] = mfma16(av, __builtin_bit_cast(bf16x8, bv), acc[nt]);
    }
  }
  // acc[nt][i] = C[row wave*16 + 4g + i][d = nt*16 + i16]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rr0 + wave * 16 + 4 * g + i;
    if (rr >= BT) continue;
    const size_t base = ((size_t)rr * H + h) * DV;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int d = nt * 16 + i16;
      const float x = bf16_to_f32(gate[base + d]);
      const float sg = 1.f / (1.f + expf(-x));
      out[base + d] = (uint16_t)bf16_rne(acc[nt][i] * sg);
    }
  }
}

// q_latent[row][c] = sum_d q_nope[row][d] * W_UK[h][d][c]; one workgroup per
// (head, 16 rows); thread owns columns tid and tid + 256.
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_lat, int BT, int H) {
  __shared__ float qs[16][DV];
  const int h = blockIdx.x % H;
  const int rr0 = (blockIdx.x / H) * 16;
  const int tid = threadIdx.x;
  for (int e = tid; e < 16 * DV; e += kThreads) {
    const int r = e / DV, d = e % DV;
    const int rr = rr0 + r;
    qs[r][d] = rr < BT ? bf16_to_f32(q_nope[((size_t)rr * H + h) * DV + d]) : 0.f;
  }
  __syncthreads();
  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc0[r] = acc1[r] = 0.f;
  const uint16_t* wh = w_uk + (size_t)h * DV * D;
  for (int d = 0; d < DV; ++d) {
    const float w0 = bf16_to_f32(wh[d * D + tid]);
    const float w1 = bf16_to_f32(wh[d * D + tid + 256]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc0[r] = fmaf(qs[r][d], w0, acc0[r]);
      acc1[r] = fmaf(qs[r][d], w1, acc1[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = rr0 + r;
    if (rr >= BT) break;
    uint16_t* dst = q_lat + ((size_t)rr * H + h) * D;
    dst[tid] = (uint16_t)bf16_rne(acc0[r]);
    dst[tid + 256] = (uint16_t)bf16_rne(acc1[r]);
  }
}

// ------------------------------------------------------------------ host side
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950 ready, -1 other

int ensure_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (ok) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(verify_attn_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AttnSmem)) != hipSuccess ||
          hipFuncSetAttribute(reinterpret_cast<const void*>(gated_epilogue_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024) != hipSuccess)
        return MLA_ERR_HIP;
    }
    st = ok ? 1 : -1;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MLA_OK : MLA_ERR_DEVICE;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int run_attention(const mla_verify_params* p, const mla::Plan& pl, const mla_bf16* q,
                  const mla_bf16* pool, const int32_t* bt, const int32_t* bounds, mla_bf16* out_lat,
                  float* lse, void* ws, hipStream_t stream) {
  AttnArgs a{};
  a.q = q;
  a.pool = pool;
  a.bt = bt;
  a.bounds = bounds;
  a.B = p->batch;
  a.T = p->q_len;
  a.H = p->num_heads;
  a.R = pl.rows;
  a.P = p->max_pages_per_req;
  a.N = p->num_pool_pages;
  a.S = pl.splits;
  a.row_tiles = pl.row_tiles;
  a.scale_log2 = p->sm_scale * kLog2e;
  a.direct = pl.use_partials ? 0 : 1;
  const size_t total_rows = (size_t)p->batch * pl.rows;
  if (pl.use_partials) {
    a.part_o = static_cast<float*>(ws);
    a.part_lse = a.part_o + (size_t)pl.splits * total_rows * D;
  } else {
    a.out_lat = out_lat;
    a.lse = lse;
  }
  const size_t items = (size_t)p->batch * pl.row_tiles * pl.splits;
  const unsigned grid = (unsigned)((items + mla::kNumXCDs - 1) / mla::kNumXCDs * mla::kNumXCDs);
  hipLaunchKernelGGL(verify_attn_kernel, dim3(grid), dim3(kThreads), sizeof(AttnSmem), stream, a);
  return launch_status();
}

bool any_null(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x == nullptr) return true;
  return false;
}
bool any_misaligned(std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x != nullptr && !mla::aligned16(x)) return true;
  return false;
}

}  // namespace

extern "C" {

int mla_verify_attn(const mla_verify_params* p, const mla_bf16* q_latent,
                    const mla_bf16* latent_kv_pages, const int32_t* block_table,
                    const int32_t* kv_bounds, mla_bf16* out_latent, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (any_null({q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse})) return MLA_ERR_NULL;
  if (any_misaligned({q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse, workspace}))
    return MLA_ERR_ARG;
  const mla::Plan pl = mla::make_plan(p, false);
  if (pl.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < pl.workspace_bytes))
    return MLA_ERR_WORKSPACE;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_attention(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse,
                     workspace, st);
  if (rc != MLA_OK || !pl.use_partials) return rc;
  const int rows = p->batch * pl.rows;
  const float* part_o = static_cast<const float*>(workspace);
  const float* part_lse = part_o + (size_t)pl.splits * rows * D;
  hipLaunchKernelGGL(combine_kernel, dim3((rows + 3) / 4), dim3(kThreads), 0, st, part_o, part_lse,
                     out_latent, lse, rows, pl.splits);
  return launch_status();
}

int mla_verify_attn_gated(const mla_verify_params* p, const mla_bf16* q_latent,
                          const mla_bf16* latent_kv_pages, const int32_t* block_table,
                          const int32_t* kv_bounds, const mla_bf16* w_uv,
                          const mla_bf16* gate_logits, mla_bf16* out, float* lse,
                          mla_bf16* out_latent, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (any_null({q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse}))
    return MLA_ERR_NULL;
  if (any_misaligned({q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                      out_latent, workspace}))
    return MLA_ERR_ARG;
  const mla::Plan pl = mla::make_plan(p, true);
  if (workspace == nullptr || workspace_bytes < pl.workspace_bytes) return MLA_ERR_WORKSPACE;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = run_attention(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, nullptr, nullptr,
                     workspace, st);
  if (rc != MLA_OK) return rc;
  const int bt_rows = p->batch * p->q_len;
  const int rows = bt_rows * p->num_heads;
  const float* part_o = static_cast<const float*>(workspace);
  const float* part_lse = part_o + (size_t)pl.splits * rows * D;
  const unsigned grid = (unsigned)(((bt_rows + 63) / 64) * p->num_heads);
  hipLaunchKernelGGL(gated_epilogue_kernel, dim3(grid), dim3(kThreads), 64 * 1024, st, part_o,
                     part_lse, w_uv, gate_logits, out, lse, out_latent, bt_rows, p->num_heads,
                     pl.splits);
  return launch_status();
}

int mla_verify_absorb_q(const mla_verify_params* p, const mla_bf16* q_nope, const mla_bf16* w_uk,
                        mla_bf16* q_latent, void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (any_null({q_nope, w_uk, q_latent})) return MLA_ERR_NULL;
  if (any_misaligned({q_nope, w_uk, q_latent})) return MLA_ERR_ARG;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  const int bt_rows = p->batch * p->q_len;
  const unsigned grid = (unsigned)(((bt_rows + 15) / 16) * p->num_heads);
  hipLaunchKernelGGL(absorb_q_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     q_nope, w_uk, q_latent, bt_rows, p->num_heads);
  return launch_status();
}

}  // extern "C"
