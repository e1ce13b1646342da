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
//   attn_kernel<MODE, KV8>  one workgroup (4 waves) per (request, row tile,
//                        KV split); tiles of 32 or 64 folded rows; a bf16
//                        or (KV8) an fp8 E4M3 latent cache, whose codes are
//                        converted exactly to bf16 for the MFMAs.  The
//                        split's pages stream HBM -> LDS by LDS-DMA
//                        (XOR-swizzled 16-byte chunks) in 64-key units, the
//                        next ones in flight while one is computed.
//                        S^T = K Q^T on bf16 MFMA 16x16x32 with Q^T held in
//                        registers; each row masked by its own bound; softmax
//                        against a per-row reference max fixed on the split's
//                        first unit (exp2 domain, fp32 sums); P in bf16 through
//                        a small LDS tile; O^T += V^T P^T on MFMA with V^T read
//                        by transposing LDS reads and O^T in accumulation
//                        registers.  Writes bf16 o_lat + lse directly (one
//                        split), or normalised bf16 partials + fp32 partial
//                        lse (split-KV).
//   attn_rows_kernel<KV8>  the same for 128-row tiles, every wave owning 32
//                        rows for QK, softmax and PV (P stays in registers);
//                        32-key units; balanced chunks of units per workgroup
//                        when the tiles are split.
//   combine_kernel       LSE merge of the S partials of every row (rows with
//                        no visible key in any split give (-inf, 0)); after
//                        the contiguous layout with small partials, each
//                        request is merged on the XCD whose L2 holds them.
//   gated_epilogue_kernel  per (head, 16 rows): LSE merge reading only the
//                        partials with a nonzero weight, then W_UV (512 -> 128)
//                        on MFMA and the sigmoid gate; optional o_lat output;
//                        small grids stage W_UV[h] in LDS during the merge.
//   absorb_q_kernel      q_latent = W_UK[h]^T q_nope on bf16 MFMA (fp32
//                        accumulate, bf16 out), W_UK[h] staged in LDS.
// The paged-cache updates (KV append, trim) live in mla_kv_update.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "mla_launch.h"
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

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// fp32 -> bf16, round to nearest even, on the hardware converter
// (v_cvt_pk_bf16_f32): two values per instruction, lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
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
  const void* pool;        // [N, 64, 512] bf16, or fp8 E4M3 codes
  const int32_t* bt;       // [B, P]
  const int32_t* bounds;   // [B, T]
  uint16_t* out_lat;       // [B, R, 512] (direct mode)
  float* lse;              // [B, R]      (direct mode)
  uint16_t* part_o;        // [S, B*R, 512] bf16 (split mode)
  float* part_lse;         // [S, B*R]
  int B, T, H, R, P, N, S, row_tiles;
  float scale_log2;        // sm_scale * log2(e)
  int direct;              // 1: write out_lat/lse, 0: write partials
  int min_split_pages;     // a split holds at least this many pages (m)
  float kv_scale;          // fp8 cache: latent = kv_scale * code value (1 for bf16)
  int l2_partials;         // partials use plain stores (they stay in the XCD's L2 for the combine)
  int balanced;            // 128-row bf16 tiles: balanced chunks of units per workgroup group
  int chunk_min;           // balanced chunks: at least this many units per chunk
};

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Eight fp8 (OCP E4M3) codes, bytes 0-3 of w0 then of w1, to eight bf16 on
// the hardware converter (two per instruction).  Every E4M3 value is exact in
// bf16; the cache's scale is applied in fp32 elsewhere (scores, normaliser).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
  const bf16x4_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4_t cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

constexpr int kBufBytes = 128 * 1024;                           // key-row staging buffers
constexpr int kPBytes = 10 * 1024;                              // P tile (bf16, padded rows)
constexpr int kStatFloats = 13 * 128;                           // per-row maxima, reference, sums
constexpr int kAttnSmemBytes =
    kBufBytes + kPBytes + mla::kMaxSplitPages * 4 + kStatFloats * 4 + 16;
// Softmax reference without rescaling: a row's reference max is fixed by the
// first unit in which it sees a key (O and the sums are still exactly zero
// then), and P = 2^(s - ref) may exceed 1 afterwards.  While no score exceeds
// the reference by more than kMaxJump (log2 domain) nothing can overflow
// (P <= 2^64, |O| <= 2^64 * |V| * keys); a row that jumps further makes the
// workgroup run its item a second time with every reference preset to the
// true maximum, where P <= 1.  The O tile is never touched by vector ALU
// instructions inside the key loop, which keeps it in accumulation registers.
constexpr float kMaxJump = 64.f;

// XOR swizzle of the 16-byte chunk index of a key row in LDS, a function of
// the key's low four bits.  With it, the 16 keys one K-operand read touches
// at one chunk, and the 4 (or 8) keys one transposing V read touches at one
// 32-byte pair, fall on distinct banks, for 128- and 256-byte LDS rows alike.
__device__ __forceinline__ int swz16(int k) {
  const int q = (k >> 2) & 3;
  return ((k & 3) << 1) | ((q & 1) ^ (q >> 1)) | ((q & 1) << 3);
}

// Streaming (nontemporal) 16-byte global access for data touched once per
// kernel: the split partials (written by the attention kernel, read back by
// the merge) and the final outputs.  They then neither displace the key
// pages in L2 nor leave dirty lines for the write-back at kernel end (both
// kernels measured faster this way).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// st_stream16 as inline assembly, for a store that sits next to a plain one
// to the same address in the other arm of a branch: the compiler merges such
// a pair into one store and drops the nontemporal hint.  The s_nop is the
// wait state a VALU write of the data registers needs after a 16-byte store.
__device__ __forceinline__ void st_stream16_asm(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off nt\n\ts_nop 0" ::"v"(p), "v"(v) : "memory");
}
// One 1 KiB key row HBM -> LDS without passing through registers: lane l
// fetches the 16 bytes at base + voff and the hardware writes them to LDS
// byte address lds + 16 l.  Written as inline assembly so that the compiler,
// which cannot tell the staging buffers apart, does not drain every
// outstanding load before each LDS read; the kernel waits explicitly.  The
// load carries the nontemporal hint (pages and Q are staged once per
// workgroup; with the hint all measured shapes ran faster, including those
// whose row tiles re-read a page).
__device__ __forceinline__ void dma_row16(const void* base, uint32_t voff, uint32_t lds) {
  // base and lds are the same for every lane; make that explicit (SGPR operands)
  const uint64_t bp = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
  base = reinterpret_cast<const void*>(bu);
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
// One dword per lane HBM -> LDS: lane l fetches 4 bytes at base + voff and the
// hardware writes them to LDS byte address lds + 4 l.  Same conventions as
// dma_row16.
__device__ __forceinline__ void dma_dword(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t bp = reinterpret_cast<uint64_t>(base);
  const uint64_t bu = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(bp >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bp);
  base = reinterpret_cast<const void*>(bu);
  lds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// O^T += V^T P^T for one 16x16 block, written so the accumulator is pinned to
// the accumulation registers (the 32-row O tile fills all 256 of them, and
// the compiler's register assignment otherwise shuttles it to and from
// VGPRs).  Inline assembly is invisible to the compiler's hazard tracking, so
// the instruction carries its own wait: a VALU write of an MFMA source needs
// two wait states; the other direction (MFMA result read by VALU) is covered
// by settle_acc().
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
               : "+a"(acc) : "v"(a_op), "v"(b_op));
}
// S^T += K Q^T for one 16x16 block, accumulator pinned to VGPRs (the
// accumulation registers hold the O tile).  Same two-wait-state guard.
__device__ __forceinline__ void mfma16_vacc(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
               : "+v"(acc) : "v"(a_op), "v"(b_op));
}
// Same, with the B operand (a Q^T block) held in accumulation registers: a
// 64-row Q^T tile does not fit in VGPRs next to everything else.
__device__ __forceinline__ void mfma16_vacc_aq(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
               : "+v"(acc) : "v"(a_op), "a"(b_op));
}
// The same three without the leading wait states, for an MFMA none of whose
// sources a VALU instruction can have written within the two instructions
// before it: operands straight from LDS reads, loop-invariant registers, and
// accumulators only MFMAs write.  The first MFMA of a chain after the VALU
// work that produced its operands keeps the guarded form.
__device__ __forceinline__ void mfma16_acc_nw(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a_op), "v"(b_op));
}
__device__ __forceinline__ void mfma16_vacc_nw(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a_op), "v"(b_op));
}
// The first MFMA of a chain: the accumulator input is the inline constant 0,
// so the accumulator needs no clearing (and no VALU write precedes it).
__device__ __forceinline__ void mfma16_vzero_nw(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a_op), "v"(b_op));
}
// The guarded form of mfma16_vzero_nw, for an A operand a VALU instruction
// just wrote (an fp8 key converted to bf16).
__device__ __forceinline__ void mfma16_vzero(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a_op), "v"(b_op));
}
// The same two with the B operand in accumulation registers.
__device__ __forceinline__ void mfma16_vacc_aq_nw(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a_op), "a"(b_op));
}
__device__ __forceinline__ void mfma16_vzero_aq_nw(f32x4& acc, const bf16x8& a_op, const bf16x8& b_op) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a_op), "a"(b_op));
}
// Wait states between the last MFMAs writing `acc` and a VALU access of it:
// callers settle the accumulators of the last 8 PV MFMAs in write order, so
// with the 3 issue slots of every later MFMA each is at least 24 wait states
// past its last write.
__device__ __forceinline__ void settle_acc(f32x4& acc) { asm volatile("s_nop 7" : "+a"(acc)); }

// Wait until at most `allowed` of this wave's vector-memory operations are
// outstanding and its LDS writes are done, then barrier.  Memory operations
// complete in issue order, so rounding `allowed` down (to a multiple of 8
// here) is always safe.  `allowed` must be wave-uniform.
__device__ __forceinline__ void wait_vm_barrier(int allowed) {
  switch (allowed >= 56 ? 7 : (allowed < 0 ? 0 : allowed >> 3)) {
    case 7: asm volatile("s_waitcnt vmcnt(56) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(48) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(40) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(32) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// Logical work item of a workgroup.  Hardware deals workgroups to the 8 XCDs
// round-robin (bid % 8); each XCD has its own L2.  A group is one (request,
// KV split) pair, and the row tiles of a group (which read the same pages)
// always sit in consecutive slots of one XCD.  Groups are laid out either
//   contiguous (rr == 0): each XCD takes a run of consecutive groups, so the
//       splits of a request share its Q tile in one L2; or
//   dealt (rr == 1): slot j of XCD x holds group 8 j + ((x - j) mod 8), so
//       the splits of one request land on different dies, and split s of
//       request b on die (b + s) mod 8 when S = 8: the first splits (never
//       empty) rotate over the dies, and a ragged batch spreads evenly (used
//       when a request has four or more row tiles, i.e. a large head fold:
//       there the per-die load, not the re-read of Q on every die, decides
//       the time).
// The grid is 8 * ceil(groups / 8) * row_tiles workgroups; returns -1 for the
// padding ones.
static_assert((mla::kNumXCDs & (mla::kNumXCDs - 1)) == 0, "XCD count is a power of two");
__host__ __device__ __forceinline__ bool dealt_layout(int row_tiles) { return row_tiles >= 4; }
__device__ __forceinline__ int logical_item(int bid, int n_groups, int row_tiles, int rr) {
  const int x = bid % mla::kNumXCDs, pos = bid / mla::kNumXCDs;
  const int per = (n_groups + mla::kNumXCDs - 1) / mla::kNumXCDs;   // group slots per XCD
  const int slot = pos / row_tiles;
  const int g = rr ? slot * mla::kNumXCDs + ((x - slot) & (mla::kNumXCDs - 1)) : x * per + slot;
  return g < n_groups ? g * row_tiles + pos % row_tiles : -1;
}

// Verify attention over one (request b, KV split s, row tile) work item of a
// 32- or 64-row tile (128-row tiles run attn_rows_kernel).  Four wavefronts;
// MODE picks the tile:
//   MODE 0 / 1   a tile of 32 / 64 folded rows (every row of a request with
//                R <= 64), 64-key staging units.  QK splits the unit's keys
//                between the waves (wave w: keys 16w .. +15, all rows), so
//                every latent byte is read from LDS once by the QK reads.
// PV splits the latent dims (wave w: dims 128w .. +127, all rows):
//   S = Q K^T   bf16 MFMA 16x16x32, K from LDS (ds_read_b128), Q^T in
//               registers for the whole item; masked by each row's own
//               bound; P = 2^(s - ref) in bf16 goes to a small LDS tile
//   O += P V    bf16 MFMA 16x16x32, V^T from LDS (ds_read_b64_tr_b16), P^T
//               from the tile; every O element lives in exactly one wave.
// Softmax without rescaling: every row with a visible key in this split sees
// one in unit 0 (the split's first key is visible whenever any is), so each
// row's reference max is fixed there for the whole item; P may exceed 1
// later (see kMaxJump for the second pass).
template <int MODE, bool KV8>
// The arguments the prologue needs first (the work-item decode, the bounds,
// the block table and Q) lead the list as plain scalars, so that the command
// processor preloads them into SGPRs (the library is built with a kernarg
// preload count of 10); the rest stay in the argument block and are fetched
// while the bounds are in flight.
__global__ __launch_bounds__(256) void attn_kernel(const uint16_t* q, const int32_t* bt,
                                                   const int32_t* bounds, int B, int S, int row_tiles,
                                                   int T, int H, int R, int P, AttnArgs a) {
  a.q = q;
  a.bt = bt;
  a.bounds = bounds;
  a.B = B;
  a.S = S;
  a.row_tiles = row_tiles;
  a.T = T;
  a.H = H;
  a.R = R;
  a.P = P;
  static_assert(MODE == 0 || MODE == 1, "32- and 64-row tiles");
  constexpr int NRB = MODE == 0 ? 2 : 4;        // 16-row blocks of the tile
  constexpr int RT = 16 * NRB;                  // rows per tile
  constexpr int UK = 64;                        // keys per staging unit
  constexpr int ROWB = KV8 ? 512 : 1024;        // LDS bytes per staged key row
  constexpr int UB = UK * ROWB;                 // bytes per staging unit
  constexpr int NBUF = kBufBytes / UB < 4 ? kBufBytes / UB : 4;   // units the buffers hold
  constexpr int ROWS_PW = UK / 4;               // key rows each wave stages per unit
  constexpr int PAIRS_PW = UK / 8;              // fp8: DMAs (two key rows each) per wave per unit
  constexpr int QKB = 1;                        // 16-key blocks per wave in QK
  constexpr int QRB = NRB;                      // 16-row blocks per wave in QK
  constexpr int KK = UK / 32;                   // 32-key MFMA steps per unit in PV
  constexpr int NDT = 8;                        // 16-dim blocks of O per wave
  constexpr int PPITCH = UK * 2 + 16;           // bytes per P row (padding spreads banks)
  constexpr int NSLOT = 4;                      // waves contributing to one row's sums
  static_assert(RT * PPITCH <= kPBytes, "P tile");

  extern __shared__ uint4 smem[];
  lds_u8* sb = (lds_u8*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)sb;
  lds_u8* sp = sb + kBufBytes;                   // P tile
  __attribute__((address_space(3))) int32_t* sm_pid =
      (__attribute__((address_space(3))) int32_t*)(sb + kBufBytes + kPBytes);
  lds_f32* sst = (lds_f32*)(sb + kBufBytes + kPBytes + mla::kMaxSplitPages * 4);
  lds_f32* xm = sst;                             // [4][RT] per-wave row maxima
  lds_f32* st_m = sst + 4 * RT;                  // [RT] reference per row
  lds_f32* st_lr = sst + 5 * RT;                 // [NSLOT][RT]
  lds_f32* st_le = sst + (5 + NSLOT) * RT;       // [NSLOT][RT]
  __attribute__((address_space(3))) int32_t* sm_redo =
      (__attribute__((address_space(3))) int32_t*)(sst + kStatFloats);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int g = lane >> 4, i16 = lane & 15;

  int id = logical_item(blockIdx.x, a.B * a.S, a.row_tiles, dealt_layout(a.row_tiles));
  if (id < 0) return;
  const int rt = id % a.row_tiles;
  id /= a.row_tiles;
  const int s = id % a.S;
  const int b = id / a.S;

  const int row0 = rt * RT;
  const int rows_here = min(RT, a.R - row0);
  const int max_keys = a.P * PG;
  // tile row of this lane's QK row block rb, and the first key of QK key block kb
  auto qrow = [&](int rb) { return 16 * rb + i16; };
  auto qkey = [&](int) { return 16 * w; };

  // Lane offsets of the DMA of row w + 4i (a key row of a unit, or a Q row):
  // its chunk order is swizzled by (w + 4i) & 15, which takes four values per
  // wave.
  uint32_t dvoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) dvoff[j] = 16u * (uint32_t)(lane ^ swz16((w + 4 * j) & 15));
  // fp8 key rows are 32 chunks of 16 bytes; chunk c of key k sits at chunk
  // position c ^ (k & 15) of its LDS row (k counted from the unit's first
  // key, a multiple of 16).  Lane l of a pair DMA writes position l & 31 of
  // row 2 pr + (l >> 5), so it fetches that row's chunk (l & 31) ^ (k & 15);
  // k & 15 takes two values per wave (pairs w + 4i for even and odd i).
  uint32_t dvoff8[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = 2 * (w + 4 * j) + (lane >> 5);
    dvoff8[j] = (uint32_t)((lane >> 5) * 512 + 16 * ((lane & 31) ^ (k & 15)));
  }

  // ---- the tile's bounds (lane j: token t_lo + j; at most 16 are used) and,
  // when it fits, the request's whole block-table row (the split's page range
  // is known only once the bounds are) go to LDS by DMA first, so that their
  // round trip does not wait behind the Q staging below: memory operations
  // complete in issue order per wave, and the wait further down lets only
  // the Q DMAs stay outstanding.  Addresses are clamped into the arrays.
  const int t_lo = row0 / a.H;
  const int ntok = (row0 + rows_here - 1) / a.H - t_lo + 1;
  const bool whole_row = a.P <= mla::kMaxSplitPages;
  lds_u8* const sm_bnd = sp;   // the P tile is idle until the first unit's softmax
  if (w == 0)
    dma_dword(a.bounds, (uint32_t)(b * a.T + min(t_lo + lane, a.T - 1)) * 4u, (uint32_t)(uintptr_t)sm_bnd);
  if (whole_row) {
    const int chunks = (a.P + 63) / 64;   // 64 entries per DMA
    for (int c = w; c < chunks; c += 4)
      dma_dword(a.bt + (size_t)b * a.P, (uint32_t)min(64 * c + lane, a.P - 1) * 4u,
                (uint32_t)(uintptr_t)(sm_pid + 64 * c));
  }

  // ---- every wave needs every Q row (QK splits the keys): Q^T is staged
  // through the last unit buffer: its address needs only the tile, and it is
  // in LDS by the time the first unit lands.
  // (an fp8 unit is smaller than a bf16 Q tile: Q then takes the top of the
  // staging area, and units are issued into it only after Q left)
  const uint32_t qb = KV8 ? (uint32_t)(kBufBytes - RT * 1024) : (uint32_t)(NBUF - 1) * UB;
#pragma unroll
  for (int i = 0; i < RT / 4; ++i) {
    const int r = w + 4 * i;
    const uint16_t* src = a.q + ((size_t)b * a.R + min(row0 + r, a.R - 1)) * D;
    dma_row16(src, dvoff[i & 3], lds0 + qb + (uint32_t)r * 1024u);
  }
  // the rest of the arguments, fetched together while the bounds are in flight
  asm volatile("" ::"s"(a.pool), "s"(a.out_lat), "s"(a.lse), "s"(a.part_o), "s"(a.part_lse), "s"(a.N),
               "s"(a.scale_log2), "s"(a.direct), "s"(a.min_split_pages)
               : "memory");
  // bounds and table landed in every wave (only this wave's Q DMAs, issued
  // after them, may still be outstanding)
  wait_vm_barrier(RT / 4);
  const int braw = *(const __attribute__((address_space(3))) int32_t*)(sm_bnd + 4 * lane);
  const int tb = (lane < ntok) ? clampi(braw, 0, max_keys) : 0;

  // ---- Q^T of this wave's QK rows: row-split tiles load their own rows
  // straight into registers in the pipeline prologue below, next to unit 0's
  // pages; key-split tiles move the staged tile from LDS there.
  bf16x8 qreg[QRB][16];   // qreg[rb][ks] = Q[tile row qrow(rb)][32 ks + 8 g .. +7]

  int n_tile = tb;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) n_tile = max(n_tile, __shfl_xor(n_tile, off));
  n_tile = __builtin_amdgcn_readfirstlane(n_tile);
  int L[QRB];           // bounds of this lane's QK rows
  int lmin = INT_MAX;   // smallest bound among the wave's valid QK rows
#pragma unroll
  for (int rb = 0; rb < QRB; ++rb) {
    const int r = row0 + qrow(rb);
    const int lr = __shfl(tb, min(r, a.R - 1) / a.H - t_lo);
    L[rb] = r < a.R ? lr : 0;
    if (r < a.R) lmin = min(lmin, lr);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lmin = min(lmin, __shfl_xor(lmin, off));
  lmin = __builtin_amdgcn_readfirstlane(lmin);

  // The tile's n_pg pages are cut into S' = min(S, ceil(n_pg / m)) balanced
  // splits; splits s >= S' are empty.  A short request in a ragged batch so
  // takes fewer, fuller splits instead of S slivers.
  const int n_pg = (n_tile + PG - 1) / PG;
  const int s_eff = min(a.S, max(1, (n_pg + a.min_split_pages - 1) / a.min_split_pages));
  const int p_begin = s < s_eff ? (s * n_pg) / s_eff : n_pg;
  const int p_end = s < s_eff ? ((s + 1) * n_pg) / s_eff : n_pg;   // <= kMaxSplitPages pages (host check)
  const int k_begin = p_begin * PG;
  const int k_end = min(p_end * PG, n_tile);
  const int n_units = k_end > k_begin ? (k_end - k_begin + UK - 1) / UK : 0;

  if (n_units == 0 && !a.direct) {
    // no key of this split is visible to the tile: its partial rows are the
    // identity (lse = -inf), and the merge never reads their O
    for (int r = tid; r < rows_here; r += kThreads)
      a.part_lse[(size_t)s * a.B * a.R + (size_t)b * a.R + row0 + r] = -INFINITY;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the Q staging has landed before LDS is released
    return;
  }
  if (!whole_row) {   // a table row past what LDS holds: this split's slice only
    for (int i = tid; i < p_end - p_begin; i += 256) sm_pid[i] = a.bt[b * a.P + p_begin + i];
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  const int pid0 = whole_row ? p_begin : 0;   // sm_pid index of the split's first page

  // Stage unit u into buffer u % NBUF.  Key rows past the tile's extent, and
  // rows of a page whose id is out of range, are zero-filled instead (never
  // read from the pool), so 0 * garbage never reaches the PV contraction.
  // Returns the number of DMA instructions this wave issued (rows skipped
  // above issue none), which the memory-counter waits below account for.
  // fp8: one DMA moves a pair of 512-byte key rows (2 pr, 2 pr + 1), lanes
  // 0-31 the first; a pair that straddles the tile's extent fetches its first
  // row with lanes 0-31 alone and zero-fills the second.
  // The page id of unit u as read from LDS (clamped to the split's last
  // unit); the pipeline reads it before the unit's turn to stage, so the LDS
  // round trip is not on the staging's path.
  auto pid_of = [&](int u) { return sm_pid[pid0 + ((min(u, max(n_units - 1, 0)) * UK) >> 6)]; };
  auto issue_unit = [&](int u, int pid_raw) {
    const uint32_t ub = (uint32_t)(u % NBUF) * UB;
    const int kl = u * UK;                         // key offset within the split
    const int pid = __builtin_amdgcn_readfirstlane(pid_raw);
    const bool pid_ok = (unsigned)pid < (unsigned)a.N;
    const int valid = pid_ok ? n_tile - (k_begin + kl) : 0;   // rows of the unit to fetch
    if constexpr (KV8) {
      const uint8_t* pbase8 = reinterpret_cast<const uint8_t*>(a.pool) +
                              ((size_t)(pid_ok ? pid : 0) * PG + (kl & 63)) * D;
#pragma unroll
      for (int i = 0; i < PAIRS_PW; ++i) {
        const int key0 = 2 * (w + 4 * i);          // first key row of the pair within the unit
        const uint32_t dst = ub + (uint32_t)key0 * 512u;
        if (key0 + 1 < valid) {
          dma_row16(pbase8 + key0 * D, dvoff8[i & 1], lds0 + dst);
        } else if (key0 < valid) {
          if (lane < 32) dma_row16(pbase8 + key0 * D, dvoff8[i & 1], lds0 + dst);
          else *(lds_u32x4*)(sb + dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
        } else {
          *(lds_u32x4*)(sb + dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
      int ops = 0;
#pragma unroll
      for (int i = 0; i < PAIRS_PW; ++i) ops += 2 * (w + 4 * i) < valid;
      return ops;
    }
    const uint16_t* pbase = reinterpret_cast<const uint16_t*>(a.pool) +
                            ((size_t)(pid_ok ? pid : 0) * PG + (kl & 63)) * D;
#pragma unroll 8
    for (int i = 0; i < ROWS_PW; ++i) {
      const int kap = w + 4 * i;                   // key row within the unit
      if (kap < valid) {
        dma_row16(pbase + kap * D, dvoff[i & 3], lds0 + ub + (uint32_t)kap * 1024u);
      } else {
        *(lds_u32x4*)(sb + ub + kap * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    int ops = 0;
#pragma unroll
    for (int i = 0; i < ROWS_PW; ++i) ops += (w + 4 * i) < valid;
    return ops;
  };

  // LDS byte offsets (within a unit buffer) of this lane's operand reads.
  // K rows qkey(kb) + i16, chunk 4 ks + g: qkb[ks & 3] + 64 (ks & 12) + 1024 qkey(kb)
  const int swl = swz16(i16);
  uint32_t qkb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    qkb[j] = (uint32_t)(i16 * 1024 + 64 * (j ^ (swl >> 2)) + 16 * (g ^ (swl & 3)));
  // V^T: lanes 4q..4q+3 of lane group g address key rows 8g + q (+4 for the
  // second read; +32 kk for k-step kk) at dims 16 D16 + 4 (i16 & 3).  For a
  // dim block D16 the offset is
  //   trow[hi] + 32 ((D16 & 7) ^ tsw[hi]) + 256 (D16 >> 3) + 32768 kk.
  uint32_t trow[2];
  int tsw[2];
  {
    const int q = i16 >> 2, e4 = i16 & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int k32 = 8 * g + q + 4 * hi;
      const int sv = swz16(k32 & 15);
      tsw[hi] = sv >> 1;
      trow[hi] = (uint32_t)(k32 * 1024 + 16 * ((e4 >> 1) ^ (sv & 1)) + 8 * (e4 & 1));
    }
  }
  // fp8 operands.  QK takes a k-order permuted within each pair of k-steps
  // (2j, 2j + 1): lane g holds dims 64 j + 16 g .. +7 for step 2j and
  // 64 j + 16 g + 8 .. +15 for step 2j + 1, one 16-byte read of its key row
  // (chunk 4 j + g); Q^T is loaded in the same order, so the dot products
  // are unchanged.  PV reads V^T with the 8-bit transposing read: in each
  // 16-lane group, lane 2k + h addresses key 8g + k, dims 16 D16 + 8h .. +7,
  // and lane i receives keys 8g .. 8g + 7 of dim 16 D16 + i.
  const uint32_t k8row = (uint32_t)i16 * 512u;                    // K: key qkey(kb) + i16
  const int v8key = 8 * g + (i16 >> 1);                           // V: key within a 32-key block
  const uint32_t v8off = (uint32_t)(v8key * 512 + 8 * (i16 & 1));
  // Q^T chunk read for k-step ks (bf16 Q rows staged with the swz16 order):
  // chunk 8 (ks >> 1) + 2 g + (ks & 1) of row i16 sits at position chunk ^ swl
  uint32_t q8b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    q8b[j] = (uint32_t)(i16 * 1024 + 16 * ((8 * (j >> 1) + 2 * g + (j & 1)) ^ swl));

  // P tile: this lane writes rows qrow(rb), keys qkey(kb) + 4g .. +3 and reads
  // the PV B operand P[row 16 rb + i16][32 kk + 8 g .. +7]
  const uint32_t pr_off = (uint32_t)(i16 * PPITCH + 16 * g);

  f32x4 o[NDT][NRB];   // O^T: o[dt][rb][i] = O[row 16 rb + i16][dim 128 w + 16 dt + 4 g + i]
  float mref[QRB];     // reference max of this lane's QK rows (log2 domain)
  float mtrue[QRB];    // lane's running max of its own raw scores
  float lround[QRB];   // lane share of sum of bf16(P): the weights PV applies
  float lexact[QRB];   // lane share of sum of P in fp32: the LSE
  float mpreset[QRB];
  bool jumped = false;
#pragma unroll
  for (int rb = 0; rb < QRB; ++rb) mpreset[rb] = -INFINITY;

  // row max over the 4 lane groups and the 4 waves
  auto row_reduce_max = [&](float (&m)[QRB]) {
#pragma unroll
    for (int rb = 0; rb < QRB; ++rb) {
      m[rb] = fmaxf(m[rb], __shfl_xor(m[rb], 16));
      m[rb] = fmaxf(m[rb], __shfl_xor(m[rb], 32));
    }
    if (g == 0) {
#pragma unroll
      for (int rb = 0; rb < QRB; ++rb) xm[w * RT + qrow(rb)] = m[rb];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < QRB; ++rb)
      m[rb] = fmaxf(fmaxf(xm[qrow(rb)], xm[RT + qrow(rb)]), fmaxf(xm[2 * RT + qrow(rb)], xm[3 * RT + qrow(rb)]));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // xm free again
  };

  auto compute_unit = [&](int u, int pass) {
    const uint32_t ub = (uint32_t)(u % NBUF) * UB;
    const int ukey0 = k_begin + u * UK;            // request position of the unit's first key
    // ---- S^T = K Q^T: sacc[kb][rb][i] = score(key qkey(kb) + 4g + i, row qrow(rb))
    // bf16: every chain starts from the MFMA's constant-0 accumulator input
    // and no source of a QK or PV MFMA is written by a VALU instruction (K,
    // V and P come from LDS, Q from LDS or memory), so they carry no wait
    // states; fp8 operands are converted by VALU instructions just before
    f32x4 sacc[QKB][QRB];
    if constexpr (KV8) {
#pragma unroll
      for (int kb = 0; kb < QKB; ++kb)
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    constexpr int KPG = 2;   // k-steps per operand group
    bf16x8 kop[2][KPG][QKB];
    auto load_k = [&](bf16x8 (&dst)[KPG][QKB], int grp) {
      if constexpr (KV8) {   // one 16-byte read: k-steps 2 grp and 2 grp + 1
        static_assert(KPG == 2, "fp8 K reads cover two k-steps");
#pragma unroll
        for (int kb = 0; kb < QKB; ++kb) {
          const u32x4 x = *(const lds_u32x4*)(sb + ub + 512u * qkey(kb) + k8row +
                                             16u * (uint32_t)((4 * grp + g) ^ i16));
          dst[0][kb] = fp8x8_to_bf16(x[0], x[1]);
          dst[1][kb] = fp8x8_to_bf16(x[2], x[3]);
        }
        return;
      }
#pragma unroll
      for (int e = 0; e < KPG; ++e) {
        const int ks = KPG * grp + e;
#pragma unroll
        for (int kb = 0; kb < QKB; ++kb)
          dst[e][kb] = *(const lds_bf16x8*)(sb + ub + qkb[ks & 3] + 64 * (ks & 12) + 1024 * qkey(kb));
      }
    };
    constexpr int NGRP = 16 / KPG;
    load_k(kop[0], 0);
#pragma unroll
    for (int grp = 0; grp < NGRP; ++grp) {
      if (grp + 1 < NGRP) load_k(kop[(grp + 1) & 1], grp + 1);
#pragma unroll
      for (int e = 0; e < KPG; ++e) {
        const int ks = KPG * grp + e;
#pragma unroll
        for (int kb = 0; kb < QKB; ++kb)
#pragma unroll
          for (int rb = 0; rb < QRB; ++rb) {
            if constexpr (KV8) {
              if (rb < 2) mfma16_vacc(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
              else mfma16_vacc_aq(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
            } else if (ks == 0) {
              if (rb < 2) mfma16_vzero_nw(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
              else mfma16_vzero_aq_nw(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
            } else {
              if (rb < 2) mfma16_vacc_nw(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
              else mfma16_vacc_aq_nw(sacc[kb][rb], kop[grp & 1][e][kb], qreg[rb][ks]);
            }
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // MFMA result -> VALU read: at least 11 wait states, ordered after the last
    // MFMA writing any of the score blocks
    static_assert(QKB * QRB == 2 || QKB * QRB == 4, "score blocks per wave");
    {
      f32x4* sf = &sacc[0][0];
      if constexpr (QKB * QRB == 4)
        asm volatile("s_nop 7\n\ts_nop 4" : "+v"(sf[0]), "+v"(sf[1]), "+v"(sf[2]), "+v"(sf[3]));
      else
        asm volatile("s_nop 7\n\ts_nop 4" : "+v"(sf[0]), "+v"(sf[1]));
    }
    // ---- raw scores; keys a row does not see become -inf.  A unit every
    // valid row of the wave sees in full (all but the last of a split, as a
    // rule) skips the masking: a wave-uniform test.
    float sv[QKB][QRB][4];
#pragma unroll
    for (int kb = 0; kb < QKB; ++kb)
#pragma unroll
      for (int rb = 0; rb < QRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb][rb][i] = sacc[kb][rb][i];
    if (!(ukey0 + UK <= lmin)) {
#pragma unroll
      for (int kb = 0; kb < QKB; ++kb) {
        const int key = ukey0 + qkey(kb) + 4 * g;
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[kb][rb][i] = (key + i) < L[rb] ? sv[kb][rb][i] : -INFINITY;
      }
    }
    int first = __builtin_amdgcn_readfirstlane(u == 0 ? 1 : 0);
    asm volatile("" : "+s"(first));   // opaque, so the key loop is not peeled for u == 0
    if (first) {   // fix every row's reference for the whole item (log2 domain)
      if (pass == 0) {
        float m[QRB];
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb) {
          m[rb] = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < QKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) m[rb] = fmaxf(m[rb], sv[kb][rb][i]);
        }
        row_reduce_max(m);
        // the scale is positive, so max(s) * scale == max(s * scale)
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb) mref[rb] = m[rb] * a.scale_log2;
      } else {
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb) mref[rb] = mpreset[rb];
      }
    }
    // ---- P = 2^(s * scale - ref) in bf16 into the P tile; lane sums and
    // raw maxima.  sum bf16(P) (the weights PV applies) comes from the packed
    // pairs with one dot product each; sum P in fp32 (the LSE) directly.
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
    const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < QRB; ++rb) {
      const float mu = (mref[rb] == -INFINITY) ? 0.f : mref[rb];   // no visible key: P = 0
      float sr = 0.f, se = 0.f, mt = mtrue[rb];
#pragma unroll
      for (int kb = 0; kb < QKB; ++kb) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mt = fmaxf(mt, sv[kb][rb][i]);
          p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][rb][i], a.scale_log2, -mu));   // -inf -> 0
        }
        const uint32_t lo = pack_bf16x2(p[0], p[1]), hi = pack_bf16x2(p[2], p[3]);
        sr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, lo), ones, sr, false);
        sr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, hi), ones, sr, false);
        se += (p[0] + p[1]) + (p[2] + p[3]);
        *(lds_u32x2*)(sp + qrow(rb) * PPITCH + 2 * (qkey(kb) + 4 * g)) = u32x2{lo, hi};
      }
      mtrue[rb] = mt;   // raw score
      jumped |= mt * a.scale_log2 > mref[rb] + kMaxJump;
      lround[rb] += sr;
      lexact[rb] += se;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // P tile complete
    // ---- O^T += V^T P^T over this wave's latent dims and all RT rows
    bf16x8 pop[NRB][KK];   // P[row 16 rb + i16][32 kk + 8 g .. +7]
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        pop[rb][kk] = *(const lds_bf16x8*)(sp + pr_off + rb * 16 * PPITCH + 64 * kk);
    bf16x8 vop[2][KK];
    auto load_v = [&](bf16x8 (&dst)[KK], int dt) {
      const int d16 = w * NDT + dt;
      if constexpr (KV8) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(sb + ub + 16384u * kk + v8off + 16u * (uint32_t)(d16 ^ (v8key & 15))));
          dst[kk] = fp8x8_to_bf16((uint32_t)x[0], (uint32_t)x[1]);
        }
        return;
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t base = ub + 32768u * kk + 256u * (uint32_t)(d16 >> 3);
        const uint32_t o0 = base + trow[0] + 32u * (uint32_t)((d16 & 7) ^ tsw[0]);
        const uint32_t o1 = base + trow[1] + 32u * (uint32_t)((d16 & 7) ^ tsw[1]);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o1));
        dst[kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    load_v(vop[0], 0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt + 1 < NDT) load_v(vop[(dt + 1) & 1], dt + 1);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if constexpr (KV8) mfma16_acc(o[dt][rb], vop[dt & 1][kk], pop[rb][kk]);
          else mfma16_acc_nw(o[dt][rb], vop[dt & 1][kk], pop[rb][kk]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the pipeline: NBUF - 1 units in flight ahead of the one computed.
  // A second pass runs only if some row's scores jumped past kMaxJump.
  constexpr int AHEAD = NBUF - 1;
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) o[dt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < QRB; ++rb) {
      mref[rb] = -INFINITY;
      mtrue[rb] = -INFINITY;
      lround[rb] = lexact[rb] = 0.f;
    }
    jumped = false;
    // DMA count per in-flight unit, 8 bits per unit u at bit 8 (u % NBUF)
    // (a packed register, not an indexed array, which would go to scratch)
    static_assert(NBUF <= 4 && ROWS_PW < 256, "ops ring packing");
    uint32_t ops_ring = 0;
    auto ring_get = [&](int v) { return (int)((ops_ring >> (8 * (v % NBUF))) & 0xFFu); };
    int issued = 0;       // units issued so far (uniform)
    int pid_next = pid_of(0);   // page id of unit `issued`
    auto issue_next = [&]() {
      const int ops = issue_unit(issued, pid_next);
      const uint32_t sh = 8u * (uint32_t)(issued % NBUF);
      ops_ring = __builtin_amdgcn_readfirstlane((ops_ring & ~(0xFFu << sh)) | ((uint32_t)ops << sh));
      ++issued;
      pid_next = pid_of(issued);
    };
    // The staged Q moves to the registers while unit 0 is in flight.
    const bool stage_q = pass == 0;
    if (n_units > 0) issue_next();
    if (stage_q) {
      // every wave's Q rows landed (only unit 0's DMAs may be outstanding)
      wait_vm_barrier(__builtin_amdgcn_readfirstlane(ring_get(0)));
#pragma unroll
      for (int rb = 0; rb < QRB; ++rb)
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          if (rb < 2) {
            qreg[rb][ks] = *(const lds_bf16x8*)(sb + qb + (KV8 ? q8b[ks & 3] : qkb[ks & 3]) + 64 * (ks & 12) +
                                                16384 * rb);
          } else {
            // row blocks 2, 3 live in accumulation registers (the MFMA B
            // operand reads them there); load them straight in so the
            // compiler never parks them in VGPRs
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=a"(qreg[rb][ks])
                         : "v"(lds0 + qb + (KV8 ? q8b[ks & 3] : qkb[ks & 3])), "i"(64 * (ks & 12) + 16384 * rb)
                         : "memory");
          }
        }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the Q buffer is free again
    } else {
      // The compiler counts only its own loads (bounds, page ids), not the
      // staging DMAs.  Draining everything here, where unit 0
      // has to land anyway, leaves it no reason to wait on the memory counter
      // inside the key loop, where such a wait would also stall on the
      // prefetched units.
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    }
    // unit 1 now; the pipeline then deepens by one unit per step until AHEAD
    // units are in flight (issuing them all here would hold back unit 0)
    if (issued < n_units) issue_next();
    for (int u = 0; u < n_units; ++u) {
      int newer = 0;   // DMA ops issued after unit u's
#pragma unroll
      for (int j = 1; j <= AHEAD; ++j) newer += (u + j < issued) ? ring_get(u + j) : 0;
      // unit u staged; unit u-1 no longer read (AHEAD whole units in flight
      // behind it: the common case, without the general wait's branches)
      newer = __builtin_amdgcn_readfirstlane(newer);
      constexpr int kFullOps = AHEAD * (KV8 ? PAIRS_PW : ROWS_PW);
      if (newer == kFullOps)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kFullOps) : "memory");
      else
        wait_vm_barrier(newer);
      // unit u-1's buffer is free: the unit AHEAD past u goes there; while
      // the pipeline is still filling, one more joins it
      if (issued < n_units && issued <= u + AHEAD) issue_next();
      if (issued < n_units && issued <= u + AHEAD && u > 0) issue_next();
      compute_unit(u, pass);
    }
    // MFMA write -> VALU write of the same accumulator (a second pass clears
    // the tile): 24 wait states.  The clear sits behind the branch below.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    if (pass == 1) break;
    if (tid == 0) *sm_redo = 0;
    __syncthreads();   // every wave is done with the buffers and has read the flag's old value
    if (__any(jumped) && lane == 0) *sm_redo = 1;
    __syncthreads();
    if (*sm_redo == 0) break;
    // second pass: every row's reference is its true maximum over the item
#pragma unroll
    for (int rb = 0; rb < QRB; ++rb) mpreset[rb] = mtrue[rb] * a.scale_log2;
    row_reduce_max(mpreset);
  }
  // accumulators of the last 8 PV MFMAs: 8 more wait states each, in write order
  {
    constexpr int LAST = (8 + NRB * KK - 1) / (NRB * KK);   // trailing dim blocks to settle
#pragma unroll
    for (int dt = NDT - LAST; dt < NDT; ++dt)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) settle_acc(o[dt][rb]);
  }

  // ---- row statistics: the QK waves publish (ref, sums) per row
#pragma unroll
  for (int rb = 0; rb < QRB; ++rb) {
    float lr = lround[rb], le = lexact[rb];
    lr += __shfl_xor(lr, 16);
    lr += __shfl_xor(lr, 32);
    le += __shfl_xor(le, 16);
    le += __shfl_xor(le, 32);
    if (g == 0) {
      const int row = qrow(rb);
      if (w == 0) st_m[row] = mref[rb];
      st_lr[w * RT + row] = lr;
      st_le[w * RT + row] = le;
    }
  }
  __syncthreads();

  // ---- finalize: (-inf, 0) for rows without a visible key.  The scaled bf16
  // rows are staged in the (now idle) key buffers and P tile at a pitch of
  // 1040 bytes (16 consecutive rows start on 16 different bank groups, and a
  // row's 16-dim blocks sit at fixed offsets), then leave as whole 1 KiB
  // rows, one store instruction per row.
  constexpr int SPITCH = 1040;
  static_assert(RT * SPITCH <= kBufBytes + kPBytes, "row staging");
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = rb * 16 + i16;
    float lr = 0.f, le = 0.f;
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) {
      lr += st_lr[k * RT + row];
      le += st_le[k * RT + row];
    }
    const bool empty = !(lr > 0.f);   // a visible key contributes P >= 1 (its max set the reference)
    // v_rcp_f32 (1 ulp); an fp8 cache's scale multiplies the values here
    const float inv = empty ? 0.f : (KV8 ? a.kv_scale * __builtin_amdgcn_rcpf(lr) : __builtin_amdgcn_rcpf(lr));
    lds_u8* const rowp = sb + row * SPITCH + 256 * w + 8 * g;    // dims 128 w + 4 g of the row
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f32x4 v = o[dt][rb] * inv;
      *(lds_u32x2*)(rowp + 32 * dt) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (w == 0 && g == 0 && row0 + row < a.R) {
      const size_t row_g = (size_t)b * a.R + row0 + row;
      // v_log_f32 is log2 with 1 ulp error
      const float l = empty ? -INFINITY : (st_m[row] + __builtin_amdgcn_logf(le)) * kLn2;
      if (a.direct) a.lse[row_g] = l;
      else a.part_lse[(size_t)s * a.B * a.R + row_g] = l;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // wave w stores tile rows w, w + 4, ...; a split's empty rows are skipped
  // (the merge never reads a partial whose lse is -inf).  Streaming stores,
  // except for partials that the combine reads back on the same XCD: those
  // stay in its L2 (they cost a write-back at the kernel's end, and save the
  // combine's round trip to memory).
  constexpr int RPW = RT / 4;   // rows per wave
  uint16_t* const dst0 = a.direct ? a.out_lat + ((size_t)b * a.R + row0) * D
                                  : a.part_o + ((size_t)s * a.B * a.R + (size_t)b * a.R + row0) * D;
  const int n_rows = min(RT, a.R - row0);
  bool live = false;   // lane j: does row w + 4 j get stored
  if (lane < RPW && w + 4 * lane < n_rows) {
    float lr = 0.f;
#pragma unroll
    for (int k = 0; k < NSLOT; ++k) lr += st_lr[k * RT + w + 4 * lane];
    live = a.direct || lr > 0.f;
  }
  const uint64_t live_mask = __ballot(live);
  u32x4 rowv[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = w + 4 * i;
    rowv[i] = *(const lds_u32x4*)(sb + row * SPITCH + 16 * lane);
  }
  if (a.l2_partials && !a.direct) {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if ((live_mask >> i) & 1) *reinterpret_cast<u32x4*>(dst0 + (size_t)(w + 4 * i) * D + 8 * lane) = rowv[i];
  } else {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if ((live_mask >> i) & 1) st_stream16_asm(dst0 + (size_t)(w + 4 * i) * D + 8 * lane, rowv[i]);
  }
}

#ifndef MLA_ROWS_AHEAD
#define MLA_ROWS_AHEAD 3
#endif
#ifndef MLA_ROWS_AHEAD8
#define MLA_ROWS_AHEAD8 5
#endif
#ifndef MLA_QK_CHAINS
#define MLA_QK_CHAINS 1
#endif
// Verify attention over one (request b, KV split s, 128-row tile) work item,
// bf16 or (KV8) fp8 E4M3 cache, with every wave owning 32 folded rows for the
// whole computation (wave w: tile rows 32 w .. +31).  An fp8 unit is 32 rows
// of 512 bytes staged in pairs of rows per DMA; K comes from one 16-byte read
// per key row for two k-steps (Q^T loaded in the same permuted dim order),
// V^T from the 8-bit transposing read, both converted to bf16 by hardware
// before their MFMAs; the cache's scale enters the score scale and the
// normaliser.
//   S^T = K Q^T     bf16 MFMA 16x16x32; K (16 keys x 32 dims) from LDS by
//                   ds_read_b128, Q^T of the wave's rows in registers; each
//                   row masked by its own bound.
//   P               2^(s - ref) in bf16, kept in registers: lane (g, i) of
//                   the QK output holds keys 4g .. 4g+3 and 16+4g .. 16+4g+3
//                   of row i, which is the B operand of PV when the PV
//                   contraction takes the unit's keys in that order.
//   O^T += V^T P^T  V^T (16 dims x 32 keys in the same key order) from two
//                   transposing LDS reads; O^T (512 dims x 32 rows) in the
//                   accumulation registers.
// No P crosses between waves, so the one barrier per unit is the one that
// releases a staging buffer.  Softmax as in attn_kernel: each row's reference
// max is fixed on the split's first unit (a second pass runs past kMaxJump).
template <bool KV8>
__global__ __launch_bounds__(256) void attn_rows_kernel(const uint16_t* q, const int32_t* bt,
                                                        const int32_t* bounds, int B, int S, int row_tiles,
                                                        int T, int H, int R, int P, AttnArgs a) {
  a.q = q;
  a.bt = bt;
  a.bounds = bounds;
  a.B = B;
  a.S = S;
  a.row_tiles = row_tiles;
  a.T = T;
  a.H = H;
  a.R = R;
  a.P = P;
  constexpr int RT = 128;                 // rows per tile
  constexpr int UK = 32;                  // keys per staging unit
  constexpr int ROWB = KV8 ? 512 : 1024;  // LDS bytes per staged key row
  constexpr int UB = UK * ROWB;           // bytes per staging unit
  constexpr int NBUF = kBufBytes / UB;    // staging units the buffers hold
  constexpr int ROWS_PW = UK / 4;         // key rows each wave stages per unit
  constexpr int OPS_PW = KV8 ? UK / 8 : ROWS_PW;   // DMA instructions per wave per unit (fp8: row pairs)
  constexpr int ND = 32;                  // 16-dim blocks of a row's O
  // units in flight ahead of the one computed (fp8 units are half the bytes)
  constexpr int AHEAD = KV8 ? MLA_ROWS_AHEAD8 : MLA_ROWS_AHEAD;
  constexpr int KR = 8;                   // K operands in flight (QK; fp8: raw 16-byte reads, two k-steps each)
  constexpr int KR8 = 4;
  constexpr int KCARRY = 2;               // bf16: second-half K operands the first half loads
  constexpr int VR = 8;                   // V operands in flight (PV)
  constexpr int SPITCH = 1040;            // staged output row pitch (bytes)
  static_assert(NBUF <= 8 && AHEAD < NBUF, "staging ring");
  static_assert(RT * SPITCH <= kBufBytes + kPBytes, "row staging");

  extern __shared__ uint4 smem[];
  lds_u8* sb = (lds_u8*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)sb;
  lds_u8* sp = sb + kBufBytes;
  __attribute__((address_space(3))) int32_t* sm_pid =
      (__attribute__((address_space(3))) int32_t*)(sb + kBufBytes + kPBytes);
  lds_f32* sst = (lds_f32*)(sb + kBufBytes + kPBytes + mla::kMaxSplitPages * 4);
  lds_f32* st_lr = sst;                   // [RT] row sums, for the store mask
  __attribute__((address_space(3))) int32_t* sm_redo =
      (__attribute__((address_space(3))) int32_t*)(sst + kStatFloats);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int max_keys = a.P * PG;

  // One work item: the rows of row tile rt of request b over a range of its
  // keys, results into partial slot `slot` (or the outputs, direct mode).
  // legacy: the range is split `slot` of the tile's own split partition;
  // otherwise units [ua, ub) (32 keys each) of the request.
  auto run_item = [&](int b, int rt, int slot, int ua, int ub, bool legacy) {
  const int s = slot;
  const int row0 = rt * RT;
  const int rows_here = min(RT, a.R - row0);
  __syncthreads();   // LDS of the previous item (staged rows, bounds) is free
  // lane-dependent address arithmetic is redone per item: made opaque here,
  // the compiler cannot hoist it out of the item loop, where it would stay
  // live (and spill) through the key loop
  int lane_o = threadIdx.x & 63, tid_o = threadIdx.x;
  asm volatile("" : "+v"(lane_o), "+v"(tid_o));
  const int lane = lane_o, tid = tid_o, g = lane >> 4, i16 = lane & 15;
  auto wrow = [&](int rb) { return 32 * w + 16 * rb + i16; };   // tile row of row block rb
  uint32_t dvoff[4];   // DMA lane offsets of key rows w + 4 j (chunk order swizzled by the row)
#pragma unroll
  for (int j = 0; j < 4; ++j) dvoff[j] = 16u * (uint32_t)(lane ^ swz16((w + 4 * j) & 15));

  // ---- the tile's bounds and the request's block-table row to LDS
  const int t_lo = row0 / a.H;
  const int ntok = (row0 + rows_here - 1) / a.H - t_lo + 1;
  const bool whole_row = a.P <= mla::kMaxSplitPages;
  lds_u8* const sm_bnd = sp;
  if (w == 0)
    dma_dword(a.bounds, (uint32_t)(b * a.T + min(t_lo + lane, a.T - 1)) * 4u, (uint32_t)(uintptr_t)sm_bnd);
  if (whole_row) {
    const int chunks = (a.P + 63) / 64;
    for (int c = w; c < chunks; c += 4)
      dma_dword(a.bt + (size_t)b * a.P, (uint32_t)min(64 * c + lane, a.P - 1) * 4u,
                (uint32_t)(uintptr_t)(sm_pid + 64 * c));
  }
  asm volatile("" ::"s"(a.pool), "s"(a.out_lat), "s"(a.lse), "s"(a.part_o), "s"(a.part_lse), "s"(a.N),
               "s"(a.scale_log2), "s"(a.direct), "s"(a.min_split_pages)
               : "memory");
  wait_vm_barrier(0);
  const int braw = *(const __attribute__((address_space(3))) int32_t*)(sm_bnd + 4 * lane);
  const int tb = (lane < ntok) ? clampi(braw, 0, max_keys) : 0;

  int n_tile = tb;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) n_tile = max(n_tile, __shfl_xor(n_tile, off));
  n_tile = __builtin_amdgcn_readfirstlane(n_tile);
  int L[2];
  int lmin = INT_MAX;   // smallest bound among the wave's valid rows
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = row0 + wrow(rb);
    const int lr = __shfl(tb, min(r, a.R - 1) / a.H - t_lo);
    L[rb] = r < a.R ? lr : 0;
    if (r < a.R) lmin = min(lmin, lr);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lmin = min(lmin, __shfl_xor(lmin, off));
  lmin = __builtin_amdgcn_readfirstlane(lmin);
  if (lmin == INT_MAX) lmin = 0;   // a wave of padding rows masks every key

  int k_begin, k_end;
  if (legacy) {
    const int n_pg = (n_tile + PG - 1) / PG;
    const int s_eff = min(a.S, max(1, (n_pg + a.min_split_pages - 1) / a.min_split_pages));
    const int p_begin = s < s_eff ? (s * n_pg) / s_eff : n_pg;
    const int p_end = s < s_eff ? ((s + 1) * n_pg) / s_eff : n_pg;
    k_begin = p_begin * PG;
    k_end = min(p_end * PG, n_tile);
  } else {
    k_begin = ua * UK;
    k_end = min(ub * UK, n_tile);
  }
  const int n_units = k_end > k_begin ? (k_end - k_begin + UK - 1) / UK : 0;
  const int p_first = k_begin / PG;   // first page of the range

  if (n_units == 0 && !a.direct) {
    for (int r = tid; r < rows_here; r += kThreads)
      a.part_lse[(size_t)s * a.B * a.R + (size_t)b * a.R + row0 + r] = -INFINITY;
    return;
  }
  if (!whole_row) {   // a table row past what LDS holds: this range's pages only
    const int n_pages = (k_end - 1) / PG - p_first + 1;
    for (int i = tid; i < n_pages; i += 256) sm_pid[i] = a.bt[(size_t)b * a.P + p_first + i];
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  const int pid_base = whole_row ? 0 : p_first;   // sm_pid index of page 0

  // Staging of unit u (32 keys: half a page) into buffer u % NBUF, one key
  // row per DMA instruction; wave w stages rows w + 4 i.  Rows past the
  // tile's extent and every row of an out-of-range page id are zero-filled
  // instead (never read from the pool).
  // fp8 rows: chunk c (16 bytes) of key k (0..31 within the unit) sits at
  // chunk position c ^ X(k), X(k) = (k & 15) ^ 8 (k >> 4 & 1): the 16 keys of
  // a K read, and the 8 keys {4g..4g+3, 16+4g..16+4g+3} of a transposing V
  // read, fall on distinct banks.
  auto xsw8 = [](int k) { return (k & 15) ^ (8 * ((k >> 4) & 1)); };
  uint32_t dvoff8[4];   // DMA lane offsets of the pair 2 (w + 4 i), 2 (w + 4 i) + 1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = 2 * (w + 4 * i) + (lane >> 5);
    dvoff8[i] = (uint32_t)((lane >> 5) * 512 + 16 * ((lane & 31) ^ xsw8(k)));
  }
  struct Stage {
    const uint8_t* base;    // the unit's first key row in the pool
    uint32_t buf;           // LDS byte offset of the unit's buffer
    int valid;              // rows of the unit to fetch
  };
  // The page id of unit u as read from LDS (clamped to the range's last
  // unit); the loop reads it one iteration before it stages the unit, so the
  // LDS round trip is not on the staging's path.
  auto pid_of = [&](int u) { return sm_pid[(k_begin + min(u, max(n_units - 1, 0)) * UK) / PG - pid_base]; };
  auto stage_of = [&](int u, int pid_raw) {
    Stage st;
    const int key0 = k_begin + u * UK;   // the unit's first key (a multiple of 32)
    const int pid = __builtin_amdgcn_readfirstlane(pid_raw);
    const bool pid_ok = (unsigned)pid < (unsigned)a.N;
    st.valid = pid_ok ? n_tile - key0 : 0;
    st.base = reinterpret_cast<const uint8_t*>(a.pool) + ((size_t)(pid_ok ? pid : 0) * PG + (key0 & 63)) * ROWB;
    st.buf = (uint32_t)(u % NBUF) * UB;
    return st;
  };
  // bf16: key row w + 4 i of the unit.  fp8: the pair of key rows 2 (w + 4 i)
  // and 2 (w + 4 i) + 1 in one DMA (lanes 0-31 the first); a pair cut by the
  // tile's extent fetches its first row with lanes 0-31 alone and zero-fills
  // the second.
  auto stage_row = [&](const Stage& st, int i, bool full) {
    if constexpr (KV8) {
      const int k0 = 2 * (w + 4 * i);
      const uint32_t dst = st.buf + (uint32_t)k0 * 512u;
      if (full || k0 + 1 < st.valid) {
        dma_row16(st.base + k0 * 512, dvoff8[i], lds0 + dst);
      } else if (k0 < st.valid) {
        if (lane < 32) dma_row16(st.base + k0 * 512, dvoff8[i], lds0 + dst);
        else *(lds_u32x4*)(sb + dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      } else {
        *(lds_u32x4*)(sb + dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const int kap = w + 4 * i;
      if (full || kap < st.valid)
        dma_row16(st.base + kap * 1024, dvoff[i & 3], lds0 + st.buf + (uint32_t)kap * 1024u);
      else
        *(lds_u32x4*)(sb + st.buf + kap * 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_ops = [&](const Stage& st) {   // DMA instructions this wave issues for the unit
    int ops = 0;
#pragma unroll
    for (int i = 0; i < OPS_PW; ++i) ops += (KV8 ? 2 * (w + 4 * i) : w + 4 * i) < st.valid;
    return ops;
  };

  // K operand: key 16 kb + i16, chunk 4 ks + g  ->  qkb[ks & 3] + 256 (ks >> 2) + 16384 kb
  const int swl = swz16(i16);
  uint32_t qkb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    qkb[j] = (uint32_t)(i16 * 1024 + 64 * (j ^ (swl >> 2)) + 16 * (g ^ (swl & 3)));
  // V^T operand of dim block d: lanes 4q .. 4q+3 of lane group g address
  // key 4g + q (first read) and 16 + 4g + q (second), dims 16 d + 4 (i16 & 3)
  const int vkey = 4 * g + (i16 >> 2);
  const int vsw = swz16(vkey);
  const uint32_t vrow = (uint32_t)(vkey * 1024 + 16 * (((i16 & 3) >> 1) ^ (vsw & 1)) + 8 * (i16 & 1));
  const int vtsw = vsw >> 1;

  // fp8 K: one 16-byte read of key 16 kb + i16 gives k-steps 2j and 2j+1
  // (dims 64 j + 16 g .. +7 and +8 .. +15; Q^T is loaded in the same order),
  // chunk 4 j + g at position (4 j + g) ^ i16 ^ 8 kb:
  //   8192 kb + 256 (j >> 2) + q8b[(j & 3) ^ 2 kb]
  uint32_t q8b[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
    q8b[x] = (uint32_t)(512 * i16 + 64 * (x ^ (i16 >> 2)) + 16 * (g ^ (i16 & 3)));
  // fp8 V^T of dim block d: lane 2k + h of lane group g addresses key
  // kap(k) = k < 4 ? 4g + k : 16 + 4g + k - 4, dims 16 d + 8 h .. +7; the
  // transposing 8-bit read hands lane i16 the eight keys kap(0..7) of dim
  // 16 d + i16, the key order of the P operand
  const int v8k = (i16 >> 1) < 4 ? 4 * g + (i16 >> 1) : 16 + 4 * g + (i16 >> 1) - 4;
  const uint32_t v8row = (uint32_t)(v8k * 512 + 8 * (i16 & 1));
  const int v8x = xsw8(v8k);

  bf16x8 qreg[2][16];   // Q[row wrow(rb)][32 ks + 8 g .. +7]  (fp8: the permuted k-order above)
  f32x4 o[ND][2];       // o[d][rb][i] = O[row wrow(rb)][dim 16 d + 4 g + i]
  float mref[2], mtrue[2], lround[2], lexact[2], mpreset[2];
  bool jumped = false;
  mpreset[0] = mpreset[1] = -INFINITY;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
  const bf16x2v ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T = K Q^T of unit u for the keys 16 kb .. 16 kb + 15:
  // s[rb][i] = score(key 16 kb + 4 g + i, row wrow(rb)).  after(ks) runs
  // after the MFMAs of k-step ks (VALU work that overlaps them).
  // The K operands travel in a ring of KR registers; the first KR-1 of a
  // half are loaded by k_prime() (for the first half, ahead of the unit's
  // DMA burst, so that their LDS latency passes during it).
  bf16x8 kop[KR];
  u32x4 kraw[KR8];
  auto load_k = [&](int u, int kb, int ks) {
    const uint32_t kbase = (uint32_t)(u % NBUF) * UB + 16384u * (uint32_t)kb;
    return *(const lds_bf16x8*)(sb + kbase + qkb[ks & 3] + 256 * (ks >> 2));
  };
  auto load_k8 = [&](int u, int kb, int j) {
    const uint32_t kbase = (uint32_t)(u % NBUF) * UB + 8192u * (uint32_t)kb + 256u * (uint32_t)(j >> 2);
    return *(const lds_u32x4*)(sb + kbase + q8b[(j & 3) ^ (2 * kb)]);
  };
  auto k_prime = [&](int u, int kb, int from = 0) {
    if constexpr (KV8) {
#pragma unroll
      for (int j = 0; j < KR8 - 1; ++j) kraw[j] = load_k8(u, kb, j);
    } else {
#pragma unroll
      for (int ks = 0; ks < KR - 1; ++ks)
        if (ks >= from) kop[ks] = load_k(u, kb, ks);
    }
  };
  // fp8: the same contraction, K converted from the raw reads one step
  // ahead of its MFMAs (the conversions of step j+1 run under those of step
  // j; the empty asm keeps them there), so no MFMA waits for a conversion
  auto qk_half8 = [&](int u, int kb, f32x4 (&s)[2], auto&& after) {
    f32x4 acc[2];
    bf16x8 kc0 = fp8x8_to_bf16(kraw[0][0], kraw[0][1]);
    bf16x8 kc1 = fp8x8_to_bf16(kraw[0][2], kraw[0][3]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + KR8 - 1 < 8) kraw[(j + KR8 - 1) % KR8] = load_k8(u, kb, j + KR8 - 1);
      const bf16x8 k0 = kc0, k1 = kc1;
      if (j + 1 < 8) {
        const u32x4 r = kraw[(j + 1) % KR8];
        kc0 = fp8x8_to_bf16(r[0], r[1]);
        kc1 = fp8x8_to_bf16(r[2], r[3]);
        asm volatile("" : "+v"(kc0), "+v"(kc1));
      }
      if (j == 0) {
        mfma16_vzero(acc[0], k0, qreg[0][0]);
        mfma16_vzero_nw(acc[1], k0, qreg[1][0]);
      } else {
        mfma16_vacc_nw(acc[0], k0, qreg[0][2 * j]);
        mfma16_vacc_nw(acc[1], k0, qreg[1][2 * j]);
      }
      after(2 * j);
      mfma16_vacc_nw(acc[0], k1, qreg[0][2 * j + 1]);
      mfma16_vacc_nw(acc[1], k1, qreg[1][2 * j + 1]);
      after(2 * j + 1);
    }
    asm volatile("s_nop 7\n\ts_nop 4" : "+v"(acc[0]), "+v"(acc[1]));
    s[0] = acc[0];
    s[1] = acc[1];
  };
  // (bf16: the first half's last steps also load the second half's first
  // KCARRY operands into the ring slots they free, so the second half does
  // not start behind all of their LDS latency; 16 is a multiple of KR, so
  // step ks of the second half finds its operand in slot ks % KR.  Carrying
  // more than two keeps too many registers live between the halves.)
  auto qk_half = [&](int u, int kb, f32x4 (&s)[2], auto&& after) {
    if constexpr (KV8) {
      qk_half8(u, kb, s, after);
      return;
    }
    static_assert(16 % KR == 0, "ring slots continue across the halves");
    // MLA_QK_CHAINS accumulator chains per row block (k-step ks feeds chain
    // ks % chains); each chain starts from a zero accumulator input
    constexpr int CH = MLA_QK_CHAINS;
    f32x4 acc[2][CH];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + KR - 1 < 16) kop[(ks + KR - 1) % KR] = load_k(u, kb, ks + KR - 1);
      else if (kb == 0 && ks + KR - 1 - 16 < KCARRY)
        kop[(ks + KR - 1) % KR] = load_k(u, 1, ks + KR - 1 - 16);
      if (ks < CH) {
        mfma16_vzero_nw(acc[0][ks % CH], kop[ks % KR], qreg[0][ks]);
        mfma16_vzero_nw(acc[1][ks % CH], kop[ks % KR], qreg[1][ks]);
      } else {
        mfma16_vacc_nw(acc[0][ks % CH], kop[ks % KR], qreg[0][ks]);
        mfma16_vacc_nw(acc[1][ks % CH], kop[ks % KR], qreg[1][ks]);
      }
      after(ks);
    }
    // MFMA result -> VALU read: at least 11 wait states after the last MFMA
    if constexpr (CH == 1) {
      asm volatile("s_nop 7\n\ts_nop 4" : "+v"(acc[0][0]), "+v"(acc[1][0]));
      s[0] = acc[0][0];
      s[1] = acc[1][0];
    } else {
      asm volatile("s_nop 7\n\ts_nop 4" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));
      s[0] = acc[0][0] + acc[0][1];
      s[1] = acc[1][0] + acc[1][1];
    }
  };

  // Raw scores of a key half with the keys a row does not see at -inf (a
  // unit every valid row of the wave sees in full skips the masking).
  auto masked = [&](int u, int kb, const f32x4 (&s)[2], float (&sv)[2][4]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[rb][i] = s[rb][i];
    const int ukey0 = k_begin + u * UK;
    if (!(ukey0 + UK <= lmin)) {
      const int key = ukey0 + 16 * kb + 4 * g;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[rb][i] = (key + i) < L[rb] ? sv[rb][i] : -INFINITY;
    }
  };

  // Softmax of one key half, in 16 steps that can ride between MFMAs:
  // score k >> 1 on even k (P = 2^(s scale - ref) overwrites it), the bf16
  // packing of a finished pair on odd k (word 2 kb + i/2 of row block rb's
  // PV operand), with the lane sums of bf16(P) (the weights) and of P (the
  // LSE) and the lane's raw maximum.
  float mu[2], mt[2], se[2], sr[2];
  u32x4 pcur[2];   // P operands (bf16 pairs) of the unit
  auto sm_step = [&](int kb, float (&sv)[2][4], int k) {
    const int j = k >> 1;
    const int rb = j >> 2, i = j & 3;
    if ((k & 1) == 0) {
      mt[rb] = fmaxf(mt[rb], sv[rb][i]);
      sv[rb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[rb][i], a.scale_log2, -mu[rb]));
    } else if (i & 1) {
      const uint32_t w2 = pack_bf16x2(sv[rb][i - 1], sv[rb][i]);
      pcur[rb][2 * kb + (i >> 1)] = w2;
      sr[rb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w2), ones, sr[rb], false);
      se[rb] += sv[rb][i - 1] + sv[rb][i];
    }
  };

  // O^T += V^T P^T of unit u over all 512 dims of the wave's 32 rows.  The
  // second row block's P is still being formed when PV starts: mid(j), the
  // VALU work that finishes it, rides the first row block's MFMAs of dim
  // blocks 0..7 (the V operands of those eight stay in registers for the
  // second row block), then the ring of VR operands runs as usual.
  static_assert(VR == 8, "the first eight V operands fill the ring");
  auto pv = [&](int u, auto&& mid) {
    const uint32_t ub = (uint32_t)(u % NBUF) * UB;
    if constexpr (KV8) {
      // raw 8-byte transposing reads (eight keys of one dim), converted to
      // bf16 right before their MFMAs; VR raw reads in flight
      auto load_v8 = [&](int d) {
        const uint32_t off = ub + v8row + 256u * (uint32_t)(d >> 4) + 16u * (uint32_t)((d & 15) ^ v8x);
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sb + off));
      };
      // each operand is converted one dim block ahead of its MFMAs
      i32x2 vraw[VR];
      bf16x8 vop[VR];
      auto cvt_v = [&](int slot) {
        const bf16x8 v = fp8x8_to_bf16((uint32_t)vraw[slot][0], (uint32_t)vraw[slot][1]);
        return v;
      };
#pragma unroll
      for (int d = 0; d < VR; ++d) vraw[d] = load_v8(d);
      vop[0] = cvt_v(0);
      vraw[0] = load_v8(VR);
#pragma unroll
      for (int d = 0; d < VR; ++d) {
        if (d + 1 < VR) {
          vop[d + 1] = cvt_v(d + 1);
          asm volatile("" : "+v"(vop[d + 1]));
          vraw[d + 1] = load_v8(d + 1 + VR);
        }
        if (d == 0)   // P of row block 0 was just packed
          mfma16_acc(o[d][0], vop[d], __builtin_bit_cast(bf16x8, pcur[0]));
        else
          mfma16_acc_nw(o[d][0], vop[d], __builtin_bit_cast(bf16x8, pcur[0]));
        mid(d);
        __builtin_amdgcn_sched_barrier(0);   // keep mid(d) between these MFMAs
      }
#pragma unroll
      for (int d = 0; d < VR; ++d) {
        if (d == 0)   // P of row block 1 was just packed by mid()
          mfma16_acc(o[d][1], vop[d], __builtin_bit_cast(bf16x8, pcur[1]));
        else
          mfma16_acc_nw(o[d][1], vop[d], __builtin_bit_cast(bf16x8, pcur[1]));
      }
      // vraw[k] holds dim block VR + k
      bf16x8 vc = cvt_v(0);
      vraw[0] = load_v8(2 * VR);
#pragma unroll
      for (int d = VR; d < ND; ++d) {
        const bf16x8 v = vc;
        if (d + 1 < ND) {
          vc = cvt_v((d + 1) % VR);
          asm volatile("" : "+v"(vc));
          if (d + 1 + VR < ND) vraw[(d + 1) % VR] = load_v8(d + 1 + VR);
        }
        mfma16_acc_nw(o[d][0], v, __builtin_bit_cast(bf16x8, pcur[0]));
        mfma16_acc_nw(o[d][1], v, __builtin_bit_cast(bf16x8, pcur[1]));
      }
      return;
    }
    auto load_v = [&](int d) {
      const uint32_t o0 = ub + vrow + 256u * (uint32_t)(d >> 3) + 32u * (uint32_t)((d & 7) ^ vtsw);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o0 + 16384));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vop[VR];
#pragma unroll
    for (int d = 0; d < VR; ++d) vop[d] = load_v(d);
#pragma unroll
    for (int d = 0; d < VR; ++d) {
      if (d == 0)   // P of row block 0 was just packed by VALU instructions
        mfma16_acc(o[d][0], vop[d], __builtin_bit_cast(bf16x8, pcur[0]));
      else
        mfma16_acc_nw(o[d][0], vop[d], __builtin_bit_cast(bf16x8, pcur[0]));
      mid(d);
      __builtin_amdgcn_sched_barrier(0);   // keep mid(d) between these MFMAs
    }
#pragma unroll
    for (int d = 0; d < VR; ++d) {
      if (d == 0)   // P of row block 1 was just packed by mid()
        mfma16_acc(o[d][1], vop[d], __builtin_bit_cast(bf16x8, pcur[1]));
      else
        mfma16_acc_nw(o[d][1], vop[d], __builtin_bit_cast(bf16x8, pcur[1]));
      if (d >= 1) vop[d - 1] = load_v(d - 1 + VR);   // both row blocks are done with dim block d-1
    }
    // slots 0..VR-2 hold dim blocks VR..2VR-2, slot VR-1 is free
#pragma unroll
    for (int d = VR; d < ND; ++d) {
      if (d + VR - 1 < ND) vop[(d + VR - 1) % VR] = load_v(d + VR - 1);
      mfma16_acc_nw(o[d][0], vop[d % VR], __builtin_bit_cast(bf16x8, pcur[0]));
      mfma16_acc_nw(o[d][1], vop[d % VR], __builtin_bit_cast(bf16x8, pcur[1]));
    }
  };

  // ---- the pipeline.  Iteration u: wait for unit u (and for every wave to
  // be done with iteration u-1), issue the DMAs of unit u+AHEAD (into the
  // buffer unit u-1 released at the barrier), QK(u) in two key halves with
  // the softmax of the first half between the MFMAs of the second,
  // softmax(u) of the second half, PV(u).
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      o[d][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      o[d][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      mref[rb] = -INFINITY;
      mtrue[rb] = -INFINITY;
      lround[rb] = lexact[rb] = 0.f;
    }
    jumped = false;
    uint64_t ops_ring = 0;   // DMA count of unit v at bits 8 (v % NBUF)
    auto ring_set = [&](int v, int ops) {
      const uint32_t sh = 8u * (uint32_t)(v % NBUF);
      const uint64_t r = (ops_ring & ~(0xFFull << sh)) | ((uint64_t)ops << sh);
      ops_ring = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32)) << 32) |
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
    };
    auto ring_get = [&](int v) { return (int)((ops_ring >> (8 * (v % NBUF))) & 0xFFull); };
    auto stage_unit = [&](int v, int pid_raw) {
      const Stage st = stage_of(v, pid_raw);
      if (st.valid >= UK) {   // a whole unit: one DMA per row (pair), no per-row test
#pragma unroll
        for (int i = 0; i < OPS_PW; ++i) stage_row(st, i, true);
        ring_set(v, OPS_PW);
      } else {
#pragma unroll
        for (int i = 0; i < OPS_PW; ++i) stage_row(st, i, false);
        ring_set(v, stage_ops(st));
      }
    };
    if (pass == 0) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = min(row0 + wrow(rb), a.R - 1);
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.R + r) * D);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
          qreg[rb][ks] = __builtin_bit_cast(bf16x8, qp[KV8 ? 8 * (ks >> 1) + 2 * g + (ks & 1) : ks * 4 + g]);
      }
    }
    // units 0 .. AHEAD-1 up front.  The compiler's own loads (Q) drain with
    // unit 0, unconditionally: the compiler does not count the staging DMAs,
    // so any wait it placed for Q inside the key loop would also wait for
    // the units in flight.
    if (n_units > 0) stage_unit(0, pid_of(0));
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int v = 1; v < AHEAD && v < n_units; ++v) stage_unit(v, pid_of(v));
    int pid_next = pid_of(AHEAD);
    for (int u = 0; u < n_units; ++u) {
      int newer = 0;   // DMA instructions issued after unit u's
#pragma unroll
      for (int j = 1; j < AHEAD; ++j) newer += (u + j < n_units) ? ring_get(u + j) : 0;
      // unit u staged; iteration u-1 done everywhere (whole units in flight
      // behind it: the common case, without the general wait's branches)
      newer = __builtin_amdgcn_readfirstlane(newer);
      if (newer == (AHEAD - 1) * OPS_PW)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((AHEAD - 1) * OPS_PW) : "memory");
      else
        wait_vm_barrier(newer);
      // the unit AHEAD past u, into the buffer unit u-1 released (one burst:
      // each DMA issue stalls the wave while the memory pipeline is busy, and
      // spread between the MFMAs those stalls cost more)
      k_prime(u, 0);
      if (u + AHEAD < n_units) stage_unit(u + AHEAD, pid_next);
      pid_next = pid_of(u + AHEAD + 1);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        mt[rb] = mtrue[rb];
        se[rb] = 0.f;
        sr[rb] = lround[rb];
      }
      f32x4 s0[2], s1[2];
      float sv0[2][4], sv1[2][4];
      qk_half(u, 0, s0, [](int) {});
      masked(u, 0, s0, sv0);
      int first = __builtin_amdgcn_readfirstlane(u == 0 ? 1 : 0);
      asm volatile("" : "+s"(first));   // opaque, so the key loop is not peeled for u == 0
      if (first) {
        // every row's reference for the whole item (log2 domain): the maximum
        // over the split's first unit, or the preset of a second pass
        k_prime(u, 1, KV8 ? 0 : KCARRY);
        qk_half(u, 1, s1, [](int) {});
        masked(u, 1, s1, sv1);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float m = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(sv0[rb][i], sv1[rb][i]));
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          // the scale is positive, so max(s) * scale == max(s * scale)
          mref[rb] = pass == 0 ? m * a.scale_log2 : mpreset[rb];
          mu[rb] = (mref[rb] == -INFINITY) ? 0.f : mref[rb];   // no visible key: P = 0
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) sm_step(0, sv0, k);
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) mu[rb] = (mref[rb] == -INFINITY) ? 0.f : mref[rb];
        k_prime(u, 1, KV8 ? 0 : KCARRY);
        qk_half(u, 1, s1, [&](int ks) { sm_step(0, sv0, ks); });
        masked(u, 1, s1, sv1);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) sm_step(1, sv1, k);   // row block 0
      pv(u, [&](int j) { sm_step(1, sv1, 8 + j); });   // row block 1 rides PV's first MFMAs
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        mtrue[rb] = mt[rb];
        jumped |= mt[rb] * a.scale_log2 > mref[rb] + kMaxJump;
        lround[rb] = sr[rb];
        lexact[rb] += se[rb];
      }
    }
    // MFMA write -> VALU write of the same accumulator (a second pass clears
    // the tile): 24 wait states.  The clear sits behind the branch below.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    if (pass == 1) break;
    if (tid == 0) *sm_redo = 0;
    __syncthreads();   // every wave is done with the buffers and has read the flag's old value
    if (__any(jumped) && lane == 0) *sm_redo = 1;
    __syncthreads();
    if (*sm_redo == 0) break;
    // second pass: every row's reference is its true maximum over the item
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float m = mtrue[rb] * a.scale_log2;
      m = fmaxf(m, __shfl_xor(m, 16));
      mpreset[rb] = fmaxf(m, __shfl_xor(m, 32));
    }
  }
  // accumulators of the last 8 PV MFMAs: 8 more wait states each, in write order
#pragma unroll
  for (int d = ND - 4; d < ND; ++d) {
    settle_acc(o[d][0]);
    settle_acc(o[d][1]);
  }

  // ---- finalize: row sums over the four lane groups; (-inf, 0) for rows
  // without a visible key; the scaled bf16 rows are staged in LDS at a pitch
  // of SPITCH bytes and leave as whole 1 KiB rows
  float lr[2], le[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    lr[rb] = lround[rb] + __shfl_xor(lround[rb], 16);
    lr[rb] += __shfl_xor(lr[rb], 32);
    le[rb] = lexact[rb] + __shfl_xor(lexact[rb], 16);
    le[rb] += __shfl_xor(le[rb], 32);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // every wave is done with the key buffers
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = wrow(rb);
    const bool empty = !(lr[rb] > 0.f);   // a visible key contributes P >= 1 (its max set the reference)
    // (an fp8 cache's scale multiplies the values here)
    const float inv = empty ? 0.f : (KV8 ? a.kv_scale * __builtin_amdgcn_rcpf(lr[rb]) : __builtin_amdgcn_rcpf(lr[rb]));
    lds_u8* const rowp = sb + row * SPITCH + 8 * g;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const f32x4 v = o[d][rb] * inv;
      *(lds_u32x2*)(rowp + 32 * d) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
    if (g == 0) {
      st_lr[row] = lr[rb];
      if (row0 + row < a.R) {
        const size_t row_g = (size_t)b * a.R + row0 + row;
        const float l = empty ? -INFINITY : (mref[rb] + __builtin_amdgcn_logf(le[rb])) * kLn2;
        if (a.direct) a.lse[row_g] = l;
        else a.part_lse[(size_t)s * a.B * a.R + row_g] = l;
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's rows are staged (it stores only its own)
  uint16_t* const dst0 = a.direct ? a.out_lat + ((size_t)b * a.R + row0) * D
                                  : a.part_o + ((size_t)s * a.B * a.R + (size_t)b * a.R + row0) * D;
  bool live = false;   // lane j: is row 32 w + j stored
  if (lane < 32 && 32 * w + lane < rows_here) live = a.direct || st_lr[32 * w + lane] > 0.f;
  const uint64_t live_mask = __ballot(live);
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    if (!((live_mask >> j) & 1)) continue;
    const int row = 32 * w + j;
    const u32x4 rv = *(const lds_u32x4*)(sb + row * SPITCH + 16 * lane);
    if (a.l2_partials && !a.direct)
      *reinterpret_cast<u32x4*>(dst0 + (size_t)row * D + 8 * lane) = rv;
    else
      st_stream16_asm(dst0 + (size_t)row * D + 8 * lane, rv);
  }
  };

  // ---- the work items of this workgroup.
  //   per-tile splits (!balanced): one item, (request, split, row tile) from
  //     the grid position.
  //   balanced chunks: request b has U_b = ceil(n_b / 32) units (n_b its
  //     largest bound) and takes MLA_VERIFY_ITEM_UNITS more positions ahead
  //     of them for an item's start-up (Q, bounds and table, the first
  //     units' latency, the finalize: about 27k cycles against 4.8k per
  //     unit), so that a chunk crossing many short requests gets fewer
  //     units; the requests' positions laid end to end are cut into G
  //     chunks of C positions, C = max(ceil(V / groups), chunk_min).  A group of
  //     row_tiles workgroups on one XCD (one per row tile, so the tiles of a
  //     request stream the same pages through one L2 together) takes chunk
  //     grp: for every request the chunk touches, its rows over those units,
  //     into partial slot grp - (first chunk of the request).  chunk_min keeps
  //     the chunks of one request at most S.  The group holding a request's
  //     last unit sets the LSEs of its unused slots to -inf; a request with no
  //     visible key gets -inf in every slot from the group owning its
  //     position.
  int rt = 0, grp = 0, C = 1, G = 1, lo = 0, hi = 0, b = 0, b_end = 0;
  __attribute__((address_space(3))) int32_t* s_start =
      (__attribute__((address_space(3))) int32_t*)(sp + 2048);   // request starts, past bounds and row overflow
  if (!a.balanced) {
    int id = logical_item(blockIdx.x, a.B * a.S, a.row_tiles, dealt_layout(a.row_tiles));
    if (id < 0) return;
    rt = id % a.row_tiles;
    id /= a.row_tiles;
    b = id / a.S;
    grp = id % a.S;
    b_end = b + 1;
  } else {
    const int gpx = 32 / a.row_tiles;                 // whole groups per XCD
    const int xcd = blockIdx.x % mla::kNumXCDs, pos = blockIdx.x / mla::kNumXCDs;
    rt = pos % a.row_tiles;
    if (pos / a.row_tiles >= gpx) return;
    const int n_groups = mla::kNumXCDs * gpx;
    grp = (pos / a.row_tiles) * mla::kNumXCDs + xcd;
    {   // exclusive prefix sums of U_b
      constexpr int PER = 8;   // requests per thread (B <= 2048)
      int cnt[PER];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int bq = tid * PER + j;
        int nb = 0;
        if (bq < a.B)
          for (int t = 0; t < a.T; ++t) nb = max(nb, clampi(a.bounds[(size_t)bq * a.T + t], 0, max_keys));
        const int ub = (nb + UK - 1) / UK;
        cnt[j] = ub > 0 ? ub + MLA_VERIFY_ITEM_UNITS : 0;   // start-up, then the units
        sum += cnt[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      __attribute__((address_space(3))) int32_t* wsum = s_start + 2044;   // [4], past s_start[0 .. B] (B <= 2000)
      if (lane == 63) wsum[w] = incl;
      __syncthreads();
      int base = incl - sum;
      for (int k = 0; k < w; ++k) base += wsum[k];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int bq = tid * PER + j;
        if (bq < a.B) s_start[bq] = base;
        base += cnt[j];
      }
      if (tid == 255) s_start[a.B] = base;
      __syncthreads();
    }
    const int U = __builtin_amdgcn_readfirstlane(s_start[a.B]);
    C = max((U + n_groups - 1) / n_groups, a.chunk_min);
    G = max(1, (U + C - 1) / C);
    if (grp >= G) return;
    lo = grp * C;
    hi = grp == G - 1 ? INT_MAX : lo + C;
    // first request with units past lo, or starting at or after lo
    int bn = a.B;
    while (b < bn) {
      const int mid = (b + bn) >> 1;
      const int s1 = __builtin_amdgcn_readfirstlane(s_start[mid + 1]);
      const int s0 = __builtin_amdgcn_readfirstlane(s_start[mid]);
      if (s1 > lo || s0 >= lo) bn = mid;
      else b = mid + 1;
    }
    b_end = a.B;
  }
  auto clear_slots = [&](int bb, int from) {   // lse = -inf in slots from .. S-1 of tile (bb, rt)
    const int row0 = rt * RT, rows_here = min(RT, a.R - row0);
    for (int i = tid; i < (a.S - from) * rows_here; i += kThreads) {
      const int sl = from + i / rows_here, r = i % rows_here;
      a.part_lse[(size_t)sl * a.B * a.R + (size_t)bb * a.R + row0 + r] = -INFINITY;
    }
  };
  for (; b < b_end; ++b) {
    int slot = grp, ua = 0, ub = 0, tail = a.S;
    if (a.balanced) {
      const int st = __builtin_amdgcn_readfirstlane(s_start[b]);
      if (st >= hi) break;
      const int Vb = __builtin_amdgcn_readfirstlane(s_start[b + 1]) - st;
      if (Vb == 0) {
        if (min(st / C, G - 1) == grp) clear_slots(b, 0);
        continue;
      }
      const int su = st + MLA_VERIFY_ITEM_UNITS;   // position of the request's first unit
      const int Ub = Vb - MLA_VERIFY_ITEM_UNITS;
      if (hi <= su) break;                           // this chunk holds only its start-up share
      slot = grp - su / C;
      ua = max(lo - su, 0);
      ub = min(hi - su, Ub);
      if (hi - su >= Ub) tail = slot + 1;   // this group holds the request's last unit
    }
    run_item(b, rt, slot, ua, ub, !a.balanced);
    if (tail < a.S) clear_slots(b, tail);
  }
}

// LSE merge of the S partials of one row, computed by one wave (lane owns
// dims 8*lane .. 8*lane+7).  Returns the row's lse; (-inf, 0) when no split
// saw a key.  A partial whose LSE is -inf gets weight 0 through a select, so
// its (possibly stale) workspace bytes never reach the sum.
//   S <= 16: every lane loads the S LSEs itself (one address per load across
//           the wave) next to its 16 bytes of each partial, all in one round
//           trip, and forms max, weights and sum in its own registers: no
//           cross-lane reduction on the path.  exp and log run on the
//           hardware's base-2 units (v_exp_f32, v_log_f32, 1 ulp).
//   S > 16: lane s fetches split s's LSE, the weights are reduced across
//           lanes, and the partials stream in batches of 16.
template <int F>   // loads in the first batch: 4 when S <= 4, else 8
__device__ __forceinline__ float merge_row(const uint16_t* __restrict__ part_o,
                                           const float* __restrict__ part_lse, int S,
                                           size_t stride_rows, size_t row, int lane, float out[8]) {
  if (S <= 16) {
    const int sl = S - 1;
    float lj[16];
    uint4 v[16];
    // split indices clamped to a valid one: the loads are unconditional and
    // issue back to back; a second batch only when there are more than 8
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const size_t r = (size_t)min(j, sl) * stride_rows + row;
      lj[j] = part_lse[r];
      v[j] = ld_stream16(part_o + r * D + lane * 8);
    }
#pragma unroll
    for (int j = F; j < 8; ++j) {
      lj[j] = -INFINITY;
      v[j] = make_uint4(0, 0, 0, 0);
    }
    if (S > 8) {
#pragma unroll
      for (int j = 8; j < 16; ++j) {
        const size_t r = (size_t)min(j, sl) * stride_rows + row;
        lj[j] = part_lse[r];
        v[j] = ld_stream16(part_o + r * D + lane * 8);
      }
    } else {
#pragma unroll
      for (int j = 8; j < 16; ++j) {
        lj[j] = -INFINITY;
        v[j] = make_uint4(0, 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = j < S ? fmaxf(mx, lj[j]) : mx;
    if (mx == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
      return -INFINITY;
    }
    float wj[16], total = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      wj[j] = j < S ? __builtin_amdgcn_exp2f((lj[j] - mx) * kLog2e) : 0.f;   // exp(-inf) = 0
      total += wj[j];
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= 8 && S <= 8) break;   // uniform
      const bool use = wj[j] > 0.f;
      const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += use ? wj[j] * bf16_to_f32(wd[e] & 0xFFFFu) : 0.f;
        acc[2 * e + 1] += use ? wj[j] * bf16_to_f32(wd[e] >> 16) : 0.f;
      }
    }
    const float inv = __builtin_amdgcn_rcpf(total);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = acc[e] * inv;
    return mx + __builtin_amdgcn_logf(total) * kLn2;
  }
  constexpr int CH = 16;   // partials in flight per lane
  const float l = (lane < S) ? part_lse[(size_t)lane * stride_rows + row] : -INFINITY;
  uint4 v[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j)
    v[j] = j < S ? ld_stream16(part_o + ((size_t)j * stride_rows + row) * D + lane * 8) : make_uint4(0, 0, 0, 0);
  float mx = l;
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (mx == -INFINITY) {
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = 0.f;
    return -INFINITY;
  }
  const float wl = (l == -INFINITY) ? 0.f : expf(l - mx);   // this lane's split weight
  float total = wl;
  for (int off = 32; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    if (s0 > 0) {   // more than 16 splits: next batch
#pragma unroll
      for (int j = 0; j < CH; ++j)
        v[j] = s0 + j < S
                   ? ld_stream16(part_o + ((size_t)(s0 + j) * stride_rows + row) * D + lane * 8)
                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float ws = __shfl(wl, (s0 + j) & 63);
      const bool use = s0 + j < S && ws > 0.f;
      const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += use ? ws * bf16_to_f32(wd[e] & 0xFFFFu) : 0.f;
        acc[2 * e + 1] += use ? ws * bf16_to_f32(wd[e] >> 16) : 0.f;
      }
    }
  }
  const float inv = 1.f / total;
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = acc[j] * inv;
  return mx + logf(total);
}

template <int F>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           uint16_t* __restrict__ out_lat,
                                                           float* __restrict__ lse, int rows, int S,
                                                           int R, int per) {
  const int lane = threadIdx.x & 63;
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (R > 0) {
    // after the contiguous attention layout (XCD x ran groups x per .. +per-1,
    // group = request * S + split): XCD x merges the requests whose first
    // split it ran, so most partials it reads were written through its L2
    const int x = blockIdx.x % mla::kNumXCDs;
    const int b_lo = (x * per + S - 1) / S;
    const int b_hi = min(rows / R, ((x + 1) * per + S - 1) / S);
    row = b_lo * R + (blockIdx.x / mla::kNumXCDs) * 4 + (threadIdx.x >> 6);
    if (row >= b_hi * R) return;
  }
  if (row >= rows) return;
  float v[8];
  const float l = merge_row<F>(part_o, part_lse, S, (size_t)rows, (size_t)row, lane, v);
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  st_stream16(out_lat + (size_t)row * D + lane * 8, w);
  if (lane == 0) lse[row] = l;
}

// Gated epilogue: workgroups of 8 waves, each owning one head h and a run of
// consecutive 64-row blocks of it ((b, t) rows 64 blk .. +63).
//   W_UV   wave w holds the MFMA B operand of out dims 16 w .. +15 of W_UV[h]
//          in registers (16 KiB per wave), loaded once per workgroup.
//   merge  wave w owns tile rows w, w + 8, ..., w + 56 of a block and merges
//          them in units of G = 64 / LPR rows (LPR >= S lanes per row): one
//          load of the unit's LSEs (one split per lane), the weights
//          exp(lse_s - max), then only the (row, split) pairs with a nonzero
//          weight are fetched, in row order, 16 per lane at a time.  A row's
//          normalised sum goes to the LDS tile as bf16 (and to out_latent),
//          its lse to memory; rows with no visible key give (-inf, 0).
//   W_UV   out[64 rows][16 dims of wave w] = tile . W_UV[h]^T on MFMA (four
//          independent 16-row accumulators), times sigmoid(gate).
// Software pipeline: the LSEs of unit u + 2 and the pairs of unit u + 1 are
// in flight while unit u is summed and its block goes through the MFMAs.
// Every global load is unconditional, from a clamped or repeated address,
// so that the count of loads in flight is static and the compiler's waits
// name exactly the loads they need.
constexpr int kEpiRows = 64;
constexpr int kEpiThreads = 512;
constexpr int kEpiPairs = 16;   // pair loads in flight per lane
// v from lane `src` (wave-uniform index)
__device__ __forceinline__ float lane_f32(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}
template <int LPR>
__global__ __launch_bounds__(kEpiThreads, 1) void gated_epilogue_kernel(
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
    const uint16_t* __restrict__ w_uv, const uint16_t* __restrict__ gate,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ out_latent,
    int BT, int H, int S, int blocks_per_wg) {
  constexpr int G = 64 / LPR;             // rows per unit
  constexpr int NG = 8 / G;               // units per block and wave
  constexpr uint64_t kSeg = LPR == 64 ? ~0ull : ((1ull << LPR) - 1);
  // 64 rows x 64 chunks of 16 bytes; chunk c of row r at r*64 + (c ^ (r & 15))
  __shared__ uint4 tile[kEpiRows * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.x % H;
  const int n_blk = (BT + kEpiRows - 1) / kEpiRows;
  const int blk0 = (blockIdx.x / H) * blocks_per_wg;
  const int n_units = (min(n_blk, blk0 + blocks_per_wg) - blk0) * NG;
  if (n_units <= 0) return;   // uniform
  const size_t rows = (size_t)BT * H;
  const int q = lane / LPR, j = lane % LPR;   // (row of the unit, split) of this lane's LSE

  // (b, t) row of row qq of unit u
  auto row_of = [&](int u, int qq) { return (blk0 + u / NG) * kEpiRows + wave + 8 * ((u % NG) * G + qq); };
  auto tile_row = [&](int u, int qq) { return wave + 8 * ((u % NG) * G + qq); };
  // this lane's LSE of unit u as loaded (clamped address; units past the
  // end read the last one), and the -inf to add where the lane holds no
  // (row, split): added when the weights are formed rather than selected at
  // the load, which the compiler would turn into a branch around the load
  // or a wait for it (a stored lse is never +inf)
  auto lse_load = [&](int u) {
    const int rr = row_of(min(u, n_units - 1), q);
    return part_lse[(size_t)min(j, S - 1) * rows + (size_t)min(rr, BT - 1) * H + h];
  };
  auto lse_mask = [&](int u) { return (row_of(u, q) < BT && j < S) ? 0.f : -INFINITY; };
  // gate of this lane's outputs of block b: row 16 rb + 4 g + i, dim 16
  // wave + i16 (loaded after the stores of the block before)
  uint32_t gb[4][4];
  auto load_gates = [&](int b) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = min((blk0 + b) * kEpiRows + 16 * rb + 4 * g + i, BT - 1);
        gb[rb][i] = gate[((size_t)rr * H + h) * DV + 16 * wave + i16];
      }
  };

  // per unit: the LSE state and the pairs in flight
  float l_raw = lse_load(0);
  float mx, wl, total;
  uint64_t m_all, m_rest;
  uint4 v[kEpiPairs];
  int bits[kEpiPairs];
  auto weights = [&](int u) {
    const float l = l_raw + lse_mask(u);
    mx = l;
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    wl = (l == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((l - mx) * kLog2e);
    total = wl;
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) total += __shfl_xor(total, off);
    m_all = __ballot(wl > 0.f);   // bit q * LPR + j: pair (row q, split j) has weight
    m_rest = m_all;
  };
  // the next (up to) kEpiPairs pairs of unit u; past the last pair a load
  // repeats the previous address and its bits entry is -1
  auto issue = [&](int u) {
    // (branch free: a branch around the address would make the compiler
    // wait for each load at the join)
    size_t off = 0;   // element offset of the pair's row, uniform
#pragma unroll
    for (int k = 0; k < kEpiPairs; ++k) {
      const int bit = __builtin_ffsll((long long)m_rest) - 1;   // -1: no pair left
      m_rest &= m_rest - 1;
      bits[k] = bit;
      const int b2 = max(bit, 0);
      const size_t o2 = ((size_t)(b2 % LPR) * rows + (size_t)row_of(u, b2 / LPR) * H + h) * D;
      off = bit >= 0 ? o2 : off;
      v[k] = ld_stream16(part_o + off + lane * 8);
    }
  };

  // prologue: the W_UV operand and the gates of block 0 go out behind the
  // LSEs of unit 0 (the scheduling barrier keeps them ahead of the wait for
  // those LSEs), then the pairs of unit 0 and the LSEs of unit 1
  const uint16_t* wd = w_uv + ((size_t)h * DV + 16 * wave + i16) * D + 8 * g;
  uint4 wreg[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) wreg[ks] = *reinterpret_cast<const uint4*>(wd + ks * 32);
  load_gates(0);
  __builtin_amdgcn_sched_barrier(0);
  weights(0);
  issue(0);
  l_raw = lse_load(1);

#pragma unroll 1
  for (int u = 0; u < n_units; ++u) {
    // ---- rows of unit u without a visible key: (-inf, 0).  Lane qq
    // collects row qq's lse; the unit's LSEs go out in one store after the
    // sums (a store per row would hold its data register, and the compiler
    // waits for the store before that register is reused)
    float lse_lane = -INFINITY;
#pragma unroll
    for (int qq = 0; qq < G; ++qq) {
      if (((m_all >> (qq * LPR)) & kSeg) != 0) continue;
      const int lr = tile_row(u, qq);
      const int rr = row_of(u, qq);
      tile[lr * 64 + (lane ^ (lr & 15))] = make_uint4(0, 0, 0, 0);
      if (out_latent && rr < BT)
        st_stream16(out_latent + ((size_t)rr * H + h) * D + lane * 8, make_uint4(0, 0, 0, 0));
    }
    // ---- weighted sums; a row is complete when the next pair belongs to another row
    int cur = -1;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    auto flush = [&]() {
      const int lr = tile_row(u, cur);
      const float tq = lane_f32(total, cur * LPR);   // > 0: the row has a pair
      const float mq = lane_f32(mx, cur * LPR);
      const float inv = __builtin_amdgcn_rcpf(tq);
      uint4 wv;
      wv.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      wv.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
      wv.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
      wv.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
      tile[lr * 64 + (lane ^ (lr & 15))] = wv;
      // (the row is below BT: it has a pair)
      if (out_latent) st_stream16(out_latent + ((size_t)row_of(u, cur) * H + h) * D + lane * 8, wv);
      lse_lane = lane == cur ? mq + __builtin_amdgcn_logf(tq) * kLn2 : lse_lane;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    };
    auto consume = [&]() {
#pragma unroll
      for (int k = 0; k < kEpiPairs; ++k) {
        if (bits[k] < 0) break;
        const int qq = bits[k] / LPR;
        if (qq != cur) {
          if (cur >= 0) flush();
          cur = qq;
        }
        const float ws = lane_f32(wl, bits[k]);
        const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += ws * bf16_to_f32(w4[e] & 0xFFFFu);
          acc[2 * e + 1] += ws * bf16_to_f32(w4[e] >> 16);
        }
      }
    };
    consume();
    while (m_rest) {   // a unit with more than kEpiPairs pairs
      issue(u);
      consume();
    }
    if (cur >= 0) flush();
    if (lane < G && row_of(u, lane) < BT) lse[(size_t)row_of(u, lane) * H + h] = lse_lane;

    // ---- the next unit's pairs and the LSEs of the one after go out now.
    // Unconditionally: after the last unit they repeat it (unused), which
    // keeps the loads in flight the same on every pass, so the compiler's
    // waits name exactly the loads they need.
    weights(min(u + 1, n_units - 1));
    issue(min(u + 1, n_units - 1));
    l_raw = lse_load(u + 2);

    // ---- block complete: out = tile . W_UV[h]^T, gated
    if (u % NG == NG - 1) {
      __syncthreads();
      // (tile rows past BT hold zeros: they are rows without a visible key)
      f32x4 acc2[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc2[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, wreg[ks]);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int r = 16 * rb + i16;
          acc2[rb] = mfma16(__builtin_bit_cast(bf16x8, tile[r * 64 + ((4 * ks + g) ^ i16)]), bv, acc2[rb]);
        }
      }
      // acc2[rb][i] = out[row 16 rb + 4 g + i of the block][dim 16 wave + i16]
      const int b = u / NG;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = (blk0 + b) * kEpiRows + 16 * rb + 4 * g + i;
          if (rr >= BT) continue;
          const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * bf16_to_f32(gb[rb][i])));
          out[((size_t)rr * H + h) * DV + 16 * wave + i16] = bf16_bits(acc2[rb][i] * sg);
        }
      load_gates(min(b + 1, n_units / NG - 1));
      __syncthreads();   // the tile is rewritten by the next block's units
    }
  }
}

// q_latent[row][c] = sum_d q_nope[row][d] * W_UK[h][d][c] on bf16 MFMA.
// One workgroup per (head h, 64-row tile, block of COLS output columns):
// the 128 x COLS block of W_UK[h] is staged into LDS by DMA as one row of
// 2 COLS bytes per d, whose 16-byte chunks are XOR-swizzled by d & 15 within
// every 256-byte group exactly as an attention key row is, so its transposed
// MFMA operand comes from the same conflict-free transposing reads as V^T
// there:
//   Q_lat^T[c][row] = sum_d W^T[c][d] Q_nope^T[d][row]
// with A = W^T blocks (16 c x 32 d) from LDS and B = q_nope blocks (32 d x
// 16 rows) straight from memory.  Wave w owns columns COLS/4 * w .. of the
// block for all 64 rows (4 k-steps).  COLS = 512 (128 KiB of LDS, 128
// MFMAs per wave) when there are enough (head, tile) items to fill the GPU;
// COLS = 128 (32 KiB, 32 MFMAs) spreads a small batch over four times as many
// workgroups.  Work items are laid out so that the workgroups of one head run
// on one XCD and share W_UK[h] in its L2.
constexpr int kAbsorbRows = 64;
template <int COLS>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                            const uint16_t* __restrict__ w_uk,
                                                            uint16_t* __restrict__ q_lat, int BT, int H) {
  static_assert(COLS == 128 || COLS == 512, "column block");
  constexpr int RB = COLS * 2;                 // bytes per staged row
  constexpr int RPD = 1024 / RB;               // rows per 1 KiB DMA
  constexpr int NCB = D / COLS;                // column blocks per head
  constexpr int NDT = COLS / 64;               // 16-column blocks per wave
  extern __shared__ uint4 smem[];
  lds_u8* const sb = (lds_u8*)smem;
  const uint32_t lds0 = (uint32_t)(uintptr_t)sb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int tiles = (BT + kAbsorbRows - 1) / kAbsorbRows;
  const int items = H * tiles * NCB;
  const int per = (items + mla::kNumXCDs - 1) / mla::kNumXCDs;   // items per XCD
  const int item = (blockIdx.x % mla::kNumXCDs) * per + blockIdx.x / mla::kNumXCDs;
  if (item >= items) return;
  const int cb = item % NCB;
  const int h = item / NCB / tiles;
  const int row0 = (item / NCB % tiles) * kAbsorbRows;

  // ---- W_UK[h][:, COLS cb .. +COLS-1] -> LDS.  DMA k moves rows RPD k ..
  // +RPD-1; wave w issues k = w + 4 i.  Lane l fetches chunk l % (64 / RPD)
  // of row RPD k + l / (64 / RPD), swizzled by that row's d & 15, which
  // depends on i only through i & 3.
  const uint16_t* wh = w_uk + (size_t)h * DV * D;
  constexpr int LPR = 64 / RPD;                // lanes per staged row
  const int lr = lane / LPR, lc = lane % LPR;  // row within the DMA, 16-byte chunk within the row
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    voff[j] = (uint32_t)(lr * (D * 2) + cb * RB +
                         16 * ((lc & ~15) | ((lc & 15) ^ swz16((RPD * (w + 4 * j) + lr) & 15))));
#pragma unroll 8
  for (int i = 0; i < DV / (4 * RPD); ++i) {
    const int k = w + 4 * i;
    dma_row16(wh + (size_t)(RPD * k) * D, voff[i & 3], lds0 + (uint32_t)k * 1024u);
  }
  // ---- q_nope^T operands of the tile, from memory meanwhile:
  // qop[rb][kk] = q_nope[row 16 rb + i16][32 kk + 8 g .. +7] (zero past BT)
  bf16x8 qop[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = row0 + 16 * rb + i16;
    const uint4* src = reinterpret_cast<const uint4*>(q_nope + ((size_t)min(row, BT - 1) * H + h) * DV);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 v = row < BT ? src[4 * kk + g] : make_uint4(0, 0, 0, 0);
      qop[rb][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMAs and loads
  __syncthreads();                       // every wave's rows of W are in LDS

  // transposing-read offsets (as for V^T in the attention kernel, d = "key")
  uint32_t trow[2];
  int tsw[2];
  {
    const int q = i16 >> 2, e4 = i16 & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int k32 = 8 * g + q + 4 * hi;
      const int sv = swz16(k32 & 15);
      tsw[hi] = sv >> 1;
      trow[hi] = (uint32_t)(k32 * RB + 16 * ((e4 >> 1) ^ (sv & 1)) + 8 * (e4 & 1));
    }
  }
  f32x4 acc[NDT][4];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[dt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int c16 = NDT * w + dt;   // 16-column block within the staged block
    bf16x8 wop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t base = (uint32_t)(32 * RB) * kk + 256u * (uint32_t)(c16 >> 3);
      const uint32_t o0 = base + trow[0] + 32u * (uint32_t)((c16 & 7) ^ tsw[0]);
      const uint32_t o1 = base + trow[1] + 32u * (uint32_t)((c16 & 7) ^ tsw[1]);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sb + o1));
      wop[kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc[dt][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[kk], qop[rb][kk], acc[dt][rb], 0, 0, 0);
  }
  // ---- acc[dt][rb][i] = q_lat[row 16 rb + i16][col COLS cb + 16 (NDT w + dt) + 4 g + i]
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = row0 + 16 * rb + i16;
    if (row >= BT) continue;
    uint16_t* dst = q_lat + ((size_t)row * H + h) * D + COLS * cb + 16 * NDT * w + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const f32x4 v = acc[dt][rb];
      *reinterpret_cast<u32x2*>(dst + 16 * dt) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

// Scratch of the allocation-free gated call: the split partials (bf16 O,
// then fp32 LSE, laid out as the workspace of mla_verify_attn_gated) of one
// call.  Every GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, never the
// device memory: host code uses the per-device address from
// hipGetSymbolAddress (g_scratch) only.
}  // namespace
static __device__ __align__(256) unsigned char scratch[MLA_VERIFY_STATIC_SCRATCH_BYTES];
namespace {

// ------------------------------------------------------------------ host side
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950 ready, -1 other
std::atomic<void*> g_scratch[kMaxDevices];      // device address of `scratch` on each GPU

int ensure_device() {
  int dev = 0;
  const hipError_t got = hipGetDevice(&dev);
  if (got == hipErrorNoDevice) return MLA_ERR_DEVICE;   // no GPU visible to this process
  if (got != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (ok) {
      const void* attn[] = {reinterpret_cast<const void*>(attn_kernel<0, false>),
                            reinterpret_cast<const void*>(attn_kernel<1, false>),
                            reinterpret_cast<const void*>(attn_kernel<0, true>),
                            reinterpret_cast<const void*>(attn_kernel<1, true>),
                            reinterpret_cast<const void*>(attn_rows_kernel<false>),
                            reinterpret_cast<const void*>(attn_rows_kernel<true>)};
      bool fail = false;
      for (const void* f : attn)
        fail |= hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kAttnSmemBytes) !=
                hipSuccess;
      fail |= hipFuncSetAttribute(reinterpret_cast<const void*>(absorb_q_kernel<512>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, DV * 512 * 2) != hipSuccess;
      // this device's copy of the static scratch (with this device current)
      void* sp = nullptr;
      fail |= hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || sp == nullptr;
      if (fail)
        return MLA_ERR_HIP;
      g_scratch[dev].store(sp, std::memory_order_release);
    }
    st = ok ? 1 : -1;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MLA_OK : MLA_ERR_DEVICE;
}

// Under the contiguous layout a request's splits run on one XCD.  When the
// partials fill at most a quarter of each XCD's L2 (the rest holds the pages
// being streamed), the attention kernel stores them without the streaming
// hint, so they stay in that L2, and the combine merges each request on the
// same XCD.
bool partials_stay_in_l2(const mla_verify_params* p, const mla::Plan& pl) {
  const size_t part_bytes_per_xcd = (size_t)pl.splits * p->batch * pl.rows * D * 2 / mla::kNumXCDs;
  return pl.splits > 1 && !pl.balanced && !dealt_layout(pl.row_tiles) &&
         part_bytes_per_xcd <= mla::kL2BytesPerXCD / 4;
}

// Launch the attention kernel.  With partials, part_o / part_lse receive the
// S split results; otherwise out_lat / lse receive the final result (S == 1).
// l2_partials: store the partials with plain stores (see partials_stay_in_l2).
int run_attention(const mla_verify_params* p, const mla::Plan& pl, const mla_bf16* q,
                  const void* pool, const int32_t* bt, const int32_t* bounds, mla_bf16* out_lat,
                  float* lse, bool partials, mla_bf16* part_o, float* part_lse, hipStream_t stream,
                  bool l2_partials = false) {
  AttnArgs a{};
  a.l2_partials = l2_partials ? 1 : 0;
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
  // an fp8 cache's scale multiplies every score (and, in the finalize, the values)
  a.kv_scale = p->kv_dtype == MLA_KV_FP8_E4M3 ? p->kv_scale : 1.0f;
  a.scale_log2 = p->sm_scale * a.kv_scale * kLog2e;
  a.min_split_pages = pl.min_split_pages;
  a.balanced = pl.balanced ? 1 : 0;
  a.chunk_min = pl.chunk_min;
  a.direct = partials ? 0 : 1;
  if (partials) {
    a.part_o = part_o;
    a.part_lse = part_lse;
  } else {
    a.out_lat = out_lat;
    a.lse = lse;
  }
  const size_t groups = (size_t)p->batch * pl.splits;
  // balanced chunks: one workgroup per CU (groups of row_tiles on one XCD)
  const unsigned grid = pl.balanced ? (unsigned)mla::kNumCUs
      : (unsigned)((groups + mla::kNumXCDs - 1) / mla::kNumXCDs * mla::kNumXCDs * pl.row_tiles);
  const int mode = pl.shape.mode;
  const bool kv8 = p->kv_dtype == MLA_KV_FP8_E4M3;
  auto go = [&](auto kernel) {
    return mla::launch(kernel, dim3(grid), dim3(kThreads), kAttnSmemBytes, stream, a.q, a.bt, a.bounds, a.B,
                       a.S, a.row_tiles, a.T, a.H, a.R, a.P, a);
  };
  if (mode == 0) return kv8 ? go(attn_kernel<0, true>) : go(attn_kernel<0, false>);
  if (mode == 1) return kv8 ? go(attn_kernel<1, true>) : go(attn_kernel<1, false>);
  if (mode == 3) return kv8 ? go(attn_rows_kernel<true>) : go(attn_rows_kernel<false>);
  return MLA_ERR_SHAPE;
}

}  // namespace

// The combine for S splits: a first batch of 4 partial loads per lane when
// S <= 4 (8 would load each partial twice), else 8.
int launch_combine(int S, dim3 grid, hipStream_t st, const mla_bf16* part_o, const float* part_lse,
                   mla_bf16* out_latent, float* lse, int rows, int R, int per) {
  auto go = [&](auto kernel) {
    return mla::launch(kernel, grid, dim3(kThreads), 0, st, part_o, part_lse, out_latent, lse, rows, S, R, per);
  };
  return S <= 4 ? go(combine_kernel<4>) : go(combine_kernel<8>);
}

namespace mla {
int device_ready() { return ensure_device(); }
}  // namespace mla

extern "C" {

int mla_verify_attn(const mla_verify_params* p, const mla_bf16* q_latent,
                    const void* latent_kv_pages, const int32_t* block_table,
                    const int32_t* kv_bounds, mla_bf16* out_latent, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse})) return MLA_ERR_NULL;
  if (mla::any_misaligned({q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse, workspace}))
    return MLA_ERR_ARG;
  const mla::Plan pl = mla::make_plan(p, false);
  if (pl.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < pl.workspace_bytes))
    return MLA_ERR_WORKSPACE;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int rows = p->batch * pl.rows;
  mla_bf16* part_o = static_cast<mla_bf16*>(workspace);
  float* part_lse = reinterpret_cast<float*>(part_o + (size_t)pl.splits * rows * D);
  const bool xcd_local = partials_stay_in_l2(p, pl);
  rc = run_attention(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, out_latent, lse,
                     pl.use_partials, part_o, part_lse, st, xcd_local);
  if (rc != MLA_OK || !pl.use_partials) return rc;
  if (xcd_local) {
    // rows grouped by the XCD that ran the request's first split
    const int per = (p->batch * pl.splits + mla::kNumXCDs - 1) / mla::kNumXCDs;
    int most = 0;
    for (int x = 0; x < mla::kNumXCDs; ++x) {
      const int b_lo = (x * per + pl.splits - 1) / pl.splits;
      const int b_hi = std::min(p->batch, ((x + 1) * per + pl.splits - 1) / pl.splits);
      most = std::max(most, (b_hi - b_lo) * pl.rows);
    }
    return launch_combine(pl.splits, dim3(mla::kNumXCDs * ((most + 3) / 4)), st, part_o, part_lse, out_latent,
                          lse, rows, pl.rows, per);
  }
  return launch_combine(pl.splits, dim3((rows + 3) / 4), st, part_o, part_lse, out_latent, lse, rows, 0, 0);
}

int mla_verify_attn_partials(const mla_verify_params* p, const mla_bf16* q_latent,
                             const void* latent_kv_pages, const int32_t* block_table,
                             const int32_t* kv_bounds, mla_bf16* part_o, float* part_lse,
                             void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({q_latent, latent_kv_pages, block_table, kv_bounds, part_o, part_lse})) return MLA_ERR_NULL;
  if (mla::any_misaligned({q_latent, latent_kv_pages, block_table, kv_bounds, part_o, part_lse}))
    return MLA_ERR_ARG;
  const mla::Plan pl = mla::make_plan(p, false);
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  return run_attention(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, nullptr, nullptr,
                       true, part_o, part_lse, static_cast<hipStream_t>(stream), partials_stay_in_l2(p, pl));
}

int mla_verify_lse_combine(int num_splits, int rows, const mla_bf16* part_o, const float* part_lse,
                           mla_bf16* out_latent, float* lse, void* stream) {
  if (num_splits < 1 || num_splits > MLA_VERIFY_MAX_SPLITS || rows < 1) return MLA_ERR_ARG;
  if (mla::any_null({part_o, part_lse, out_latent, lse})) return MLA_ERR_NULL;
  if (mla::any_misaligned({part_o, part_lse, out_latent, lse})) return MLA_ERR_ARG;
  const int rc = ensure_device();
  if (rc != MLA_OK) return rc;
  return launch_combine(num_splits, dim3((rows + 3) / 4), static_cast<hipStream_t>(stream), part_o, part_lse,
                        out_latent, lse, rows, 0, 0);
}

}  // extern "C"

namespace {
// The gated call after its host checks, with `workspace` holding at least
// pl.workspace_bytes of device memory.
int gated_call(const mla_verify_params* p, const mla::Plan& pl, const mla_bf16* q_latent,
               const void* latent_kv_pages, const int32_t* block_table, const int32_t* kv_bounds,
               const mla_bf16* w_uv, const mla_bf16* gate_logits, mla_bf16* out, float* lse,
               mla_bf16* out_latent, void* workspace, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int bt_rows = p->batch * p->q_len;
  const int rows = bt_rows * p->num_heads;
  mla_bf16* part_o = static_cast<mla_bf16*>(workspace);
  float* part_lse = reinterpret_cast<float*>(part_o + (size_t)pl.splits * rows * D);
  // the partials' store rule is the one mla_verify_attn_partials uses, so the
  // attention kernel launched on its own is the kernel of this call
  const int rc = run_attention(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, nullptr, nullptr, true,
                     part_o, part_lse, st, partials_stay_in_l2(p, pl));
  if (rc != MLA_OK) return rc;
  // one workgroup per CU when the heads leave room: a head's blocks are
  // shared among ceil(CUs / H) workgroups (W_UV[h] is loaded once per
  // workgroup), each taking a run of consecutive blocks
  const int n_blk = (bt_rows + kEpiRows - 1) / kEpiRows;
  const int wg_per_head = std::max(1, std::min(n_blk, mla::kNumCUs / p->num_heads));
  const int blocks_per_wg = (n_blk + wg_per_head - 1) / wg_per_head;
  const unsigned grid = (unsigned)(((n_blk + blocks_per_wg - 1) / blocks_per_wg) * p->num_heads);
  const int S = pl.splits;
  auto go = [&](auto kernel) {
    return mla::launch(kernel, dim3(grid), dim3(kEpiThreads), 0, st, part_o, part_lse, w_uv, gate_logits, out,
                       lse, out_latent, bt_rows, p->num_heads, S, blocks_per_wg);
  };
  if (S <= 8) return go(gated_epilogue_kernel<8>);
  if (S <= 16) return go(gated_epilogue_kernel<16>);
  if (S <= 32) return go(gated_epilogue_kernel<32>);
  return go(gated_epilogue_kernel<64>);
}

// Host checks shared by the two gated entry points.
int gated_checks(const mla_verify_params* p, const mla_bf16* q_latent, const void* latent_kv_pages,
                 const int32_t* block_table, const int32_t* kv_bounds, const mla_bf16* w_uv,
                 const mla_bf16* gate_logits, mla_bf16* out, float* lse, mla_bf16* out_latent,
                 const void* workspace) {
  const int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse}))
    return MLA_ERR_NULL;
  if (mla::any_misaligned({q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                           out_latent, workspace}))
    return MLA_ERR_ARG;
  return MLA_OK;
}
}  // namespace

extern "C" {

int mla_verify_attn_gated(const mla_verify_params* p, const mla_bf16* q_latent,
                          const void* latent_kv_pages, const int32_t* block_table,
                          const int32_t* kv_bounds, const mla_bf16* w_uv,
                          const mla_bf16* gate_logits, mla_bf16* out, float* lse,
                          mla_bf16* out_latent, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = gated_checks(p, q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                        out_latent, workspace);
  if (rc != MLA_OK) return rc;
  const mla::Plan pl = mla::make_plan(p, true);
  if (workspace == nullptr || workspace_bytes < pl.workspace_bytes) return MLA_ERR_WORKSPACE;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  return gated_call(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                    out_latent, workspace, stream);
}

int mla_verify_attn_gated_noalloc(const mla_verify_params* p, const mla_bf16* q_latent,
                                  const void* latent_kv_pages, const int32_t* block_table,
                                  const int32_t* kv_bounds, const mla_bf16* w_uv,
                                  const mla_bf16* gate_logits, mla_bf16* out, float* lse,
                                  mla_bf16* out_latent, void* stream) {
  int rc = gated_checks(p, q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                        out_latent, nullptr);
  if (rc != MLA_OK) return rc;
  const mla::Plan pl = mla::make_plan(p, true);
  if (pl.workspace_bytes > (size_t)MLA_VERIFY_STATIC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  void* ws = g_scratch[dev].load(std::memory_order_acquire);
  if (ws == nullptr) return MLA_ERR_HIP;
  // Nothing in the scratch has to start at zero: the attention kernel writes
  // every partial LSE of the call (-inf for a split that sees no key of a
  // row), and the epilogue reads a partial row only when its LSE is finite.
  return gated_call(p, pl, q_latent, latent_kv_pages, block_table, kv_bounds, w_uv, gate_logits, out, lse,
                    out_latent, ws, stream);
}

int mla_verify_absorb_q(const mla_verify_params* p, const mla_bf16* q_nope, const mla_bf16* w_uk,
                        mla_bf16* q_latent, void* stream) {
  int rc = mla::check_params(p);
  if (rc != MLA_OK) return rc;
  if (mla::any_null({q_nope, w_uk, q_latent})) return MLA_ERR_NULL;
  if (mla::any_misaligned({q_nope, w_uk, q_latent})) return MLA_ERR_ARG;
  rc = ensure_device();
  if (rc != MLA_OK) return rc;
  const int bt_rows = p->batch * p->q_len;
  // whole rows of W_UK[h] per workgroup once the (head, tile) items fill the
  // GPU; column quarters for a small batch
  const int pairs = ((bt_rows + kAbsorbRows - 1) / kAbsorbRows) * p->num_heads;
  const bool whole = pairs >= mla::kNumCUs;
  const int items = pairs * (whole ? 1 : 4);
  const unsigned grid = (unsigned)((items + mla::kNumXCDs - 1) / mla::kNumXCDs * mla::kNumXCDs);
  if (whole)
    return mla::launch(absorb_q_kernel<512>, dim3(grid), dim3(kThreads), DV * 512 * 2,
                       static_cast<hipStream_t>(stream), q_nope, w_uk, q_latent, bt_rows, p->num_heads);
  return mla::launch(absorb_q_kernel<128>, dim3(grid), dim3(kThreads), DV * 128 * 2,
                     static_cast<hipStream_t>(stream), q_nope, w_uk, q_latent, bt_rows, p->num_heads);
}

}  // extern "C"
