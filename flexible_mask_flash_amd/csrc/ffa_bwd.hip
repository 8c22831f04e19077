// gfx950 (MI355X) kernels and the C ABI call of the flexible-mask attention backward.
//
// With P = exp(scale q.k - lse) over the visible keys (the forward's weights,
// rebuilt from its lse) and an upstream gradient dO, the gradients follow from
// the softmax Jacobian:
//   dP = dO V^T,  dS = P * (dP - Dd) with Dd = rowsum(dO * O),
//   dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q
// (both pages present the forward as a differentiable training operator:
// MagiAttention quickstart, "Single-GPU Flex-Flash-Attention"; FlagAttention
// user guide, "FlashAttention").
//
// Two kernels, both on the caller's stream, no atomics (results are bitwise
// reproducible):
//   ffa_bwd_main<D, 0>   dQ, query-major: a workgroup owns the rows of one
//                        forward item (unsplit) and walks its key tiles; it
//                        first forms -Dd and L of its rows and stores them into
//                        the workspace (every (row, head) is in one such item)
//   ffa_bwd_main<D, 1>   dK and dV, key-major: a workgroup owns 128 keys of one
//                        kv head and walks the query tiles of the transposed
//                        slices once per query head of that kv head
// Both main kernels are one template: a lane owns one "row" (a query for dQ, a
// key for dK/dV) whose operand fragments stay in registers (q and dO, or k or v),
// and 64-row tiles of the other side stream through LDS (k and v, or q and dO),
// filled by global_load_lds (double-buffered query-major, triple-buffered
// key-major).  Per tile:
//   X1 = A F1^T, X2 = B F2^T       (v_mfma_f32_32x32x16_bf16, A/B rows from LDS)
//   P = exp2(X1 c2 - L), dS = P (X2 - Dd)   (fp32)
// Key-major, the lane's 32 scores belong to 32 different queries, each with its own
// L and Dd: rather than holding those in registers, the MFMAs start their
// accumulators from them (X1 from -lse / scale, X2 from -Dd, read from LDS), so that
// P = exp2(c2 X1) and dS = P X2 directly.
//   dQ^T += K^T dS (query-major); dV^T += dO^T P and dK^T += Q^T dS (key-major, one
//   product in each wave of a pair)
// with the transposed operands read from LDS by ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <string>
#include <type_traits>

#include "ffa_device.h"

// A named namespace: the D <= 32 instances of ffa_bwd_main are compiled in
// ffa_bwd_small.hip (which includes this file with FFA_BWD_KERNELS_ONLY set), with
// other scheduler flags, and must be the same entities in both objects.
namespace ffa::bwd {

using namespace ffa::dev;
using ffa::kBlockN;
using ffa::kItemRec;
using ffa::kRec;

constexpr float kLog2e = 1.44269504088896340736f;

struct PreArgs {
  const __bf16* out;
  const __bf16* dout;
  const float* lse;
  float* lw;  // [batch][heads_q][total_q]: L (see below)
  float* dw;  // [batch][heads_q][total_q]: -Dd
  int64_t o_sb, o_st, o_sh;
  int64_t d_sb, d_st, d_sh;
  int64_t l_sb, l_st, l_sh;
  int32_t total_q, heads_q;
  float scale;  // softmax_scale
  int32_t fold;  // L = -lse / scale (uncapped) instead of lse * log2 e (soft-capped)
};

struct BwdArgs {
  const int32_t* items;
  const int32_t* runs;
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int64_t q_sb, q_st, q_sh;
  int64_t k_sb, k_st, k_sh;
  int64_t v_sb, v_st, v_sh;
  int64_t d_sb, d_st, d_sh;
  int64_t dq_sb, dq_st, dq_sh;
  int64_t dk_sb, dk_st, dk_sh;
  int64_t dv_sb, dv_st, dv_sh;
  float* lw;  // L and -Dd per (batch, head, row): read by the key-major kernel; the
  float* dw;  // query-major kernel writes them (from out, dout and lse) before it
  const __bf16* out;  // query-major: the forward's output and lse (for Dd and L)
  int64_t o_sb, o_st, o_sh;
  const float* lse;
  int64_t l_sb, l_st, l_sh;
  float scale_log2;  // softmax_scale * log2(e)
  float scale;
  int32_t total_q, total_k, heads_q, batch;
  int32_t heads_per_item;  // query heads per query-major item
  int32_t kv_ratio;        // heads_q / heads_kv
  float cap_log2;          // softcap * log2(e)          (CAP instances)
  float cap_arg;           // 2 * log2(e) * scale / softcap
  float* tot;              // total attention (TOT instances): tot[b*t_sb + key*t_st + h*t_sh]
  int64_t t_sb, t_st, t_sh;
};

struct SinkArgs {
  const float* sink;
  float* dsink;
  const float* lw;
  const float* dw;
  int64_t sk_sb, sk_st, sk_ss, sk_sh;
  int32_t total_q, heads_q, n_sink;
  float l_mul;  // lse * log2 e = l_mul * L
};

// tanh(y) from z = 2 y log2(e): 1 - 2 / (1 + 2^z); exact limits +-1 for +-inf
__device__ __forceinline__ float tanh_from_2ylog2e(float z) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

#ifndef FFA_BWD_KERNELS_ONLY
// d sink[b, s, h] = -sum_i exp(sink - lse[i,h]) Dd[i,h]   (shared logits, sink_st == 0)
// d sink[b, i, s, h] = -exp(sink[i] - lse[i,h]) Dd[i,h]     (per-row logits)
// One workgroup per (sink, head, batch element); the sum runs in a fixed order.
__global__ __launch_bounds__(256) void ffa_bwd_dsink(SinkArgs a) {
  const int s = blockIdx.x / a.heads_q, h = blockIdx.x % a.heads_q, b = blockIdx.y;
  const int64_t row0 = ((int64_t)b * a.heads_q + h) * a.total_q;
  const float* sp = a.sink + (int64_t)b * a.sk_sb + (int64_t)s * a.sk_ss + (int64_t)h * a.sk_sh;
  float* dp = a.dsink + (int64_t)b * a.sk_sb + (int64_t)s * a.sk_ss + (int64_t)h * a.sk_sh;
  float acc = 0.0f;
  for (int t = threadIdx.x; t < a.total_q; t += 256) {
    const float x = sp[(int64_t)t * a.sk_st] * kLog2e;
    const float c = __builtin_amdgcn_exp2f(x - a.l_mul * a.lw[row0 + t]) * a.dw[row0 + t];
    if (a.sk_st != 0) dp[(int64_t)t * a.sk_st] = c;
    else acc += c;
  }
  if (a.sk_st != 0) return;
  __shared__ float part[4];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) *dp = (part[0] + part[1]) + (part[2] + part[3]);
}
#endif  // FFA_BWD_KERNELS_ONLY

// -Dd[b,h,t] with Dd = sum_d dO[b,t,h,d] O[b,t,h,d] (fp32 from the bf16 values), and
// L[b,h,t] = -lse / scale (fold) or lse * log2 e: either way a row that sees no key
// (lse = -inf) gets the value that makes its P zero.  Total attention launches it
// for L alone (no out); the gradient's query-major kernel forms both itself, with
// the same sums in the same order.
template <int D, typename T>
__global__ __launch_bounds__(256) void ffa_bwd_pre(PreArgs a) {
  using V8 = typename ElemT<T>::v8;
  constexpr int TPP = D / 8;      // lanes per (row, head), 8 values each
  constexpr int PPB = 256 / TPP;  // (row, head) pairs per workgroup
  const int b = blockIdx.y;
  const int64_t pairs = (int64_t)a.total_q * a.heads_q;
  const int64_t p = (int64_t)blockIdx.x * PPB + threadIdx.x / TPP;
  const int c = threadIdx.x % TPP;
  float acc = 0.0f;
  int64_t t = 0;
  int h = 0;
  if (p < pairs) {
    t = p / a.heads_q;
    h = (int)(p - t * a.heads_q);
  }
  if (p < pairs && a.out) {  // no out (total attention): only L
    const V8 o = *reinterpret_cast<const V8*>(a.out + (int64_t)b * a.o_sb + t * a.o_st +
                                                          (int64_t)h * a.o_sh + c * 8);
    const V8 g = *reinterpret_cast<const V8*>(a.dout + (int64_t)b * a.d_sb + t * a.d_st +
                                                          (int64_t)h * a.d_sh + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int m = TPP / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (p < pairs && c == 0) {
    const int64_t idx = ((int64_t)b * a.heads_q + h) * a.total_q + t;
    a.dw[idx] = -acc;
    const float l = a.lse[(int64_t)b * a.l_sb + t * a.l_st + (int64_t)h * a.l_sh];
    if (a.fold) a.lw[idx] = l == -INFINITY ? -INFINITY : -l / a.scale;
    else a.lw[idx] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// LDS swizzle of tiles that are read both as MFMA A rows (16 consecutive rows,
// one 16-byte chunk each) and transposed (4 consecutive rows, two chunks, per
// 16-lane group): the XOR spreads both patterns over all bank groups, and it is
// the same for rows r and r + 16, so tiles can be addressed with compile-time
// row offsets in steps of 16 (the rows r + 8 get their own address).
template <int OFF>
__device__ __forceinline__ void lds_write_b128(uint32_t addr, f32x4_t v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}

template <int D>
__device__ __forceinline__ int swz_b(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
         : D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                   : ((r >> 2) & 3);  // 64-byte rows: four rows per bank window already
}

// Occupancy: two waves per SIMD (or more), so that one wave's VALU work hides behind
// another's MFMAs.  The query-major kernel and total attention run one wave per 32
// rows.  The key-major kernel (dK and dV) runs a pair of waves per 32-key block
// (PAIR), eight waves for the item's 128 keys: one wave per block would hold both fp32
// accumulators and both fragments (~330 registers at D = 128, one wave per SIMD).
// Role 0 holds k and dV and computes X1 = K Q^T, P and dV += P^T dO; role 1 holds v
// and dK and computes X2 = V dO^T - Dd, takes P from its partner through LDS and
// computes dS and dK += dS^T Q.  Role 1 works one step behind role 0, so the
// hand-over needs no barrier of its own and the two waves of a SIMD run their
// products and softmax work out of phase (tiles triple-buffered; one barrier per
// step as elsewhere).  Roles alternate over the wave index as (w ^ (w >> 2)) & 1, so
// that each SIMD holds one wave of each role whether the hardware places waves w
// and w + 4 or waves 2i and 2i + 1 on one SIMD; the key block is w >> 1.
template <int D, bool KV, bool TOT>
constexpr bool kPairBwd = KV && !TOT;
template <int D, bool KV, bool TOT>
constexpr int kBwdWgWaves = kPairBwd<D, KV, TOT> ? 2 * ffa::kWaves : ffa::kWaves;

// Register budget: two waves per SIMD, three for the query-major kernel at D = 64
// (167 VGPRs; +1.4% on that backward).  At D <= 32 both kernels fit four anyway.
template <int D, bool KV>
constexpr int kBwdWavesEU = (!KV && D == 64) ? 3 : 2;

// TOT (key-major only): FlagAttention's total attention, sum_i P[i,h,j] per key j and
// query head h -- the same walk over the transposed worklist with only X1 and P.
template <int D, bool KV, bool CAP, bool TOT, typename T>
__global__ __launch_bounds__((64 * kBwdWgWaves<D, KV, TOT>)) __attribute__((amdgpu_waves_per_eu(kBwdWavesEU<D, KV>, kBwdWavesEU<D, KV>))) void ffa_bwd_main(BwdArgs a) {
  using V8 = typename ElemT<T>::v8;
  using V4 = typename ElemT<T>::v4;
  using V2 = typename ElemT<T>::v2;
  (void)sizeof(V2);
  static_assert(!TOT || KV, "total attention walks the key-major worklist");
  constexpr int BN = kBlockN;          // 64 rows per streamed tile
  // D = 16 keeps its tiles in the 32-wide layout (as the forward): the row products
  // read only the 16 real head dims, the transposed reads of the unused half only
  // feed accumulator rows 16-31, which are never stored.
  constexpr int DL = D < 32 ? 32 : D;  // head dims of an LDS row and of the accumulators
  constexpr int GC = D / 8;            // 16-byte chunks of a global row
  constexpr int ROWB = DL * 2;         // bytes of one row in LDS
  constexpr int CH = DL / 8;           // 16-byte chunks per LDS row
  constexpr int KSTEPS = D / 16;       // MFMA k-steps over the head dim
  constexpr int DBLK = DL / 32;        // 32-wide head-dim blocks of the accumulators
  constexpr int TILE = BN * ROWB;      // bytes of one streamed tile
  constexpr bool PAIR = kPairBwd<D, KV, TOT>;
  constexpr int W = kBwdWgWaves<D, KV, TOT>;  // waves of the workgroup (they share the DMA)
  // PAIR: only the four role-1 waves issue the tile DMAs, so that role 0, whose
  // exponentials dominate the VALU work, spends no issue slots on the DMA setup
  constexpr int WD = PAIR ? ffa::kWaves : W;  // waves that share the DMA of a tile
  constexpr int NLD = TILE / (1024 * WD);     // DMA instructions per thread per tile
  constexpr int RPL = 1024 * WD / ROWB;       // rows between consecutive DMA instructions
  static_assert(NLD * 1024 * WD == TILE, "DMA split");
  static_assert(BN == 64 && (D == 16 || D == 32 || D == 64 || D == 128), "tile shape");
  // LDS: A0 | B0 | A1 | B1 (double-buffered tiles), then (key-major) L and Dd of
  // the 64 streamed rows per buffer, 1 KiB each (one DMA instruction writes
  // 64 x 16 bytes; the first 256 count).  The L / Dd block has its own base
  // address so that every read offset fits the 16-bit immediate.
  // PAIR (three buffers, the dS/dK wave one step behind): Q0 | Q1 | Q2, then
  // dO0 | dO1 | dO2, then L / Dd of the three steps, then two P hand-over
  // buffers of 4 KiB per 32-key block (lane l's 64 bytes as four 16-byte words
  // 1 KiB apart, so each write or read instruction is one contiguous KiB).  Each
  // role reads rows from one region and transposed tiles from the other, so its
  // two address sets each have their own base and every offset fits 16 bits.
  constexpr int BUFB = 2 * TILE;
  constexpr int LDB = KV ? 2048 : 0;
  constexpr int XB = PAIR ? 4 * 4096 : 0;
  constexpr int QREG = 0, DREG = 3 * TILE, LDREG = 6 * TILE, XREG = 6 * TILE + 3 * LDB;
  constexpr int SMEM = PAIR ? XREG + 2 * XB : 2 * BUFB + 2 * LDB;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int bid = blockIdx.x;
  const int item_idx = bid / a.batch;
  const int b = bid - item_idx * a.batch;
  const FFA_CONST int32_t* itp = (const FFA_CONST int32_t*)(a.items + (int64_t)item_idx * kItemRec);
  const int r0 = itp[0], nrows = itp[1], h0 = itp[2], run_off = itp[3], n_runs = itp[4];
  const int total_tiles = itp[6];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;
  const int G = KV ? 1 : a.heads_per_item;
  // PAIR: role 0 (k, P, dV) or 1 (v, dS, dK) and the 32-key block of the wave
  const int role = PAIR ? ((wave ^ (wave >> 2)) & 1) : 0;
  const int kw = PAIR ? wave >> 1 : wave;
  const int g = kw % G, rsub = kw / G;
  const int lrow = rsub * 32 + (lane & 31);
  const int row = r0 + lrow;
  const bool row_ok = lrow < nrows;
  const int hk = KV ? h0 : h0 / a.kv_ratio;  // kv head
  const int hq = h0 + g;                     // query head of the row (query-major)

  // ---- the row's fragments (B operands, head-dim half hh): q and dO, or k and v
  V8 f1[KSTEPS], f2[KSTEPS];
  {
    const __bf16* p1 = (PAIR && role) ? a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh + (int64_t)row * a.v_st
                       : KV ? a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh + (int64_t)row * a.k_st
                            : a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)row * a.q_st;
    const __bf16* p2 = KV ? a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh + (int64_t)row * a.v_st
                          : a.dout + (int64_t)b * a.d_sb + (int64_t)hq * a.d_sh + (int64_t)row * a.d_st;
    const bool load = row_ok && n_runs > 0;
    // query-major: dO is read for every row of the item, those without keys included,
    // since its Dd is computed below
    const bool load2 = KV ? load : row_ok;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (load) {
        f1[s] = reinterpret_cast<const V8*>(p1 + hh * (D / 2))[s];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f1[s][j] = (T)0.0f;
      }
      if (load2) {
        f2[s] = reinterpret_cast<const V8*>(p2 + hh * (D / 2))[s];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) f2[s][j] = (T)0.0f;
      }
    }
  }
  // query-major: the row's L (lse * log2 e) and -Dd are per lane.  The dQ worklist
  // holds every (row, head) exactly once, rows without keys included, so this kernel
  // also stores both into the workspace for the key-major kernel and the sink
  // gradient that run after it.  Dd = sum_d dO[d] out[d]: 16-byte chunks of 8 values
  // summed in order by FMA, then the chunk sums in a butterfly whose first level
  // pairs chunk s of the lower head-dim half with chunk s of the upper one.
  float l_row = 0.0f, d_row = 0.0f;
  if constexpr (!KV) {
    if (row_ok) {
      const V8* po = reinterpret_cast<const V8*>(a.out + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh +
                                                 (int64_t)row * a.o_st + hh * (D / 2));
      float cs[KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const V8 o = po[s];
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)f2[s][e], acc);
        cs[s] = acc;
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) cs[s] = partner_sum(cs[s]);
#pragma unroll
      for (int m = KSTEPS / 2; m >= 1; m >>= 1)
#pragma unroll
        for (int s = 0; s < m; ++s) cs[s] += cs[s + m];
      const float l = a.lse[(int64_t)b * a.l_sb + (int64_t)row * a.l_st + (int64_t)hq * a.l_sh];
      // L: -lse / scale (the K Q^T accumulators start from it), or lse * log2 e when
      // soft-capped; rows that see nothing get the value that makes P = 0
      const float lw = CAP ? (l == -INFINITY ? INFINITY : l * kLog2e) : (l == -INFINITY ? -INFINITY : -l / a.scale);
      if (hh == 0) {
        const int64_t idx = ((int64_t)b * a.heads_q + hq) * a.total_q + row;
        a.lw[idx] = lw;
        a.dw[idx] = -cs[0];
      }
      l_row = CAP ? lw : -(lw * a.scale_log2);
      d_row = -cs[0];
    }
  }

  // acc1: dQ (query-major) or the pair wave's own dV or dK (key-major)
  f32x16_t acc1[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc1[d][i] = 0.0f;

  // ---- per-lane LDS read addresses (the low 10 bits of the LDS base are zero)
  const uint32_t lds = (uint32_t)(uintptr_t)(FFA_LDS char*)smem;
  // A operand rows: row (lane & 31) (+32 for the second block), chunk (D/16) hh + s
  uint32_t r_addr[KSTEPS];
  {
    const int r = lane & 31;
    const uint32_t rbase = PAIR ? (role ? DREG : QREG) : 0;
    const uint32_t a0 = lds + rbase + r * ROWB + ((((D / 16) * hh) ^ swz_b<DL>(r)) << 4);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) r_addr[s] = a0 ^ (s << 4);
  }
  // transposed reads of head-dim block d: rows 4 hh + j/4 (lo) and 8 + 4 hh + j/4
  // (hi), +16 t; columns 32 d + 16 (grp & 1) + 4 (j & 3)
  uint32_t t_lo[DBLK], t_hi[DBLK];
  {
    const int grp = lane >> 4, jl = lane & 15;
    const int vr = 4 * hh + (jl >> 2);
    const int cl = 2 * (grp & 1) + ((jl & 3) >> 1);
    const uint32_t tbase = PAIR ? (role ? QREG : DREG) : 0;
    const uint32_t lo = lds + tbase + vr * ROWB + ((cl ^ swz_b<DL>(vr)) << 4) + (jl & 1) * 8;
    const uint32_t hi = lds + tbase + (vr + 8) * ROWB + ((cl ^ swz_b<DL>(vr + 8)) << 4) + (jl & 1) * 8;
#pragma unroll
    for (int d = 0; d < DBLK; ++d) {
      t_lo[d] = lo ^ (d << 6);
      t_hi[d] = hi ^ (d << 6);
    }
  }
  // key-major: L / Dd of rows 32 blk + 8 gq + 4 hh .. +3 are one 16-byte read
  const uint32_t ld_addr = lds + (PAIR ? LDREG : 2 * BUFB) + 16 * hh;
  // PAIR: the lane's 16-byte words of the P hand-over of its block (buffer 0)
  const uint32_t x_addr = lds + XREG + kw * 4096 + lane * 16;

  // ---- DMA of a streamed tile: as in the forward, instruction i of wave w fills
  // LDS block (W i + w); lane l's 16 bytes are chunk (lin % CH) of row (lin / CH),
  // loaded from the swizzled global chunk.  Rows past `total` re-read the last
  // row (their scores are masked).
  const int dwv = PAIR ? kw : wave;  // the wave's index among the DMA waves
  const int lin0 = dwv * 64 + lane;
  const int dr0 = lin0 / CH, dp = lin0 % CH;
  const int sw0 = swz_b<DL>(dr0);
  // D = 16: lanes whose chunk is padding load zeros (an offset past the buffer's end,
  // no memory access) or, on the last tile, chunk 0 of their row again
  const bool pad_lane = GC < CH && (dp ^ sw0) >= GC;
  auto dma = [&](const char* base, int64_t st_b, int dst_off, int kstart, int total) {
    if (kstart + BN <= total) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kstart * st_b), (short)0, 0x7fffffff, kBufferFlags);
      const uint32_t goff = pad_lane ? 0x80000000u : (uint32_t)(dr0 * st_b) + ((dp ^ sw0) << 4);
      uint32_t ldst = (uint32_t)(uintptr_t)(FFA_LDS char*)smem + dst_off + dwv * 1024;
      int32_t rstep = (int32_t)(RPL * st_b);
      asm volatile("" : "+s"(ldst), "+s"(rstep));
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FFA_LDS void*)(uintptr_t)(ldst + i * WD * 1024), 16, goff,
                                                 i * rstep, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int r = min(kstart + dr0 + i * RPL, total - 1);
        __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)r * st_b + (pad_lane ? 0 : (dp ^ sw0) << 4)),
                                         (FFA_LDS void*)(smem + dst_off + (i * WD + dwv) * 1024), 16, 0, 0);
      }
    }
  };
  // key-major: L and Dd of the 64 streamed queries, one DMA instruction each
  // (wave 0; lanes 16-63 repeat lanes 0-15 into padding).  Reads past total_q
  // return zeros (the buffer's size ends there).
  auto dma_ld = [&](int dst_off, int head, int kstart) {
    if (dwv == 0) {
      const int64_t rowoff = ((int64_t)b * a.heads_q + head) * a.total_q + kstart;
      const int nrec = max(0, a.total_q - kstart) * 4;
      const __amdgpu_buffer_rsrc_t rl =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.lw + rowoff), (short)0, nrec, kBufferFlags);
      const __amdgpu_buffer_rsrc_t rd =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.dw + rowoff), (short)0, nrec, kBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (FFA_LDS void*)(smem + dst_off), 16, (lane & 15) * 16, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FFA_LDS void*)(smem + dst_off + 1024), 16, (lane & 15) * 16, 0,
                                               0, 0);
    }
  };

  // ---- X = C + T F^T for the streamed tile T at LDS offset OFF: two 32-row blocks
  // (xa, xb); init() sets C once the LDS reads issued before the call have
  // landed, hook(m) runs after the m-th MFMA is issued
  auto rowprod = [&](auto off_tag, const V8(&f)[KSTEPS], f32x16_t& xa, f32x16_t& xb, auto&& hook, auto&& init) {
    constexpr int OFF = decltype(off_tag)::value;
    constexpr int NQ = 2 * KSTEPS;
    constexpr int KIF = NQ < 4 ? NQ : 4;  // reads in flight; no more than the tile has (D = 16: 2)
    f32x4_t rf[KIF];
    static_for<KIF>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      rf[m] = lds_read_b128<OFF + (m % 2) * 32 * ROWB>(r_addr[m / 2]);
    });
    static_for<NQ>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      constexpr int later = (m + KIF - 1 < NQ - 1) ? KIF - 1 : NQ - 1 - m;
      lds_wait<later>();
      if constexpr (m == 0) init(xa, xb);
      fence(rf[m % KIF]);
      if constexpr (m % 2 == 0)
        xa = mfma32(as_v8<T>(rf[m % KIF]), f[m / 2], xa);
      else
        xb = mfma32(as_v8<T>(rf[m % KIF]), f[m / 2], xb);
      if constexpr (m + KIF < NQ) {
        constexpr int r = m + KIF;
        rf[m % KIF] = lds_read_b128<OFF + (r % 2) * 32 * ROWB>(r_addr[r / 2]);
      }
      hook(std::integral_constant<int, m>{});
    });
  };

  // ---- acc^T += T^T X for the streamed tile T at LDS offset OFF (16 rows per
  // MFMA, the reads of step t+1 in flight during the MFMAs of step t)
  auto trprod = [&](auto off_tag, const V8(&xf)[4], f32x16_t(&acc)[DBLK], auto&& hook) {
    constexpr int OFF = decltype(off_tag)::value;
    s16x4_t vlo[2][DBLK], vhi[2][DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d) {
      vlo[0][d] = lds_read_tr16<OFF>(t_lo[d]);
      vhi[0][d] = lds_read_tr16<OFF>(t_hi[d]);
    }
    static_for<4>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      constexpr int cur = t & 1, nxt = cur ^ 1;
      if constexpr (t + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          vlo[nxt][d] = lds_read_tr16<OFF + 16 * (t + 1) * ROWB>(t_lo[d]);
          vhi[nxt][d] = lds_read_tr16<OFF + 16 * (t + 1) * ROWB>(t_hi[d]);
        }
      }
      constexpr int ahead = (t + 1 < 4) ? 2 * DBLK : 0;
      static_for<DBLK>([&](auto d_tag) {
        constexpr int d = decltype(d_tag)::value;
        lds_wait<2 * (DBLK - 1 - d) + ahead>();
        fence(vlo[cur][d]);
        fence(vhi[cur][d]);
        const s16x8_t vv = {vlo[cur][d][0], vlo[cur][d][1], vlo[cur][d][2], vlo[cur][d][3],
                            vhi[cur][d][0], vhi[cur][d][1], vhi[cur][d][2], vhi[cur][d][3]};
        acc[d] = mfma32(__builtin_bit_cast(V8, vv), xf[t], acc[d]);
      });
      hook(std::integral_constant<int, t>{});
    });
  };

  // edge mask: streamed position j (absolute) is visible from the lane's row iff
  // row + lo_base <= j < min(k_hi, row + edge_base)
  auto mask = [&](const TileIt& t, f32x16_t& xa, f32x16_t& xb) {
    const int base = t.kstart() + 4 * hh;
    const int lim = min(t.khi, row + t.eb) - base;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rel = 8 * (i >> 2) + (i & 3);
      if (rel >= lim) xa[i] = -INFINITY;
      if (rel + 32 >= lim) xb[i] = -INFINITY;
    }
    if (t.lb != -ffa::kNoEdge) {
      const int low = row + t.lb - base;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rel = 8 * (i >> 2) + (i & 3);
        if (rel < low) xa[i] = -INFINITY;
        if (rel + 32 < low) xb[i] = -INFINITY;
      }
    }
  };

  const float c2 = a.scale_log2;
  const FFA_CONST int32_t* rp = (const FFA_CONST int32_t*)(a.runs + (int64_t)run_off * kRec);
  const int64_t ast_b = KV ? a.q_st * 2 : a.k_st * 2;
  const int64_t bst_b = KV ? a.d_st * 2 : a.v_st * 2;
  const int total = KV ? a.total_q : a.total_k;
  // streamed tensors of a query head (key-major) or of the kv head (query-major)
  auto a_base = [&](int head) -> const char* {
    return KV ? (const char*)(a.q + (int64_t)b * a.q_sb + (int64_t)head * a.q_sh)
              : (const char*)(a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh);
  };
  auto b_base = [&](int head) -> const char* {
    return KV ? (const char*)(a.dout + (int64_t)b * a.d_sb + (int64_t)head * a.d_sh)
              : (const char*)(a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh);
  };

  // one step: a tile of the runs for one query head (key-major: every tile of
  // the item once per query head of the kv head)
  struct Step {
    TileIt t;
    int head, jt;
  };
  const int heads_per_step = KV ? a.kv_ratio : 1;
  const int steps = total_tiles * heads_per_step;
  auto load = [&](auto buf_tag, const Step& s) {
    constexpr int BI = decltype(buf_tag)::value;
    constexpr int OA = PAIR ? QREG + BI * TILE : BI * BUFB;
    constexpr int OB = PAIR ? DREG + BI * TILE : BI * BUFB + TILE;
    dma(a_base(s.head), ast_b, OA, s.t.kstart(), total);
    if constexpr (!TOT) dma(b_base(s.head), bst_b, OB, s.t.kstart(), total);
    if constexpr (KV) dma_ld((PAIR ? LDREG : 2 * BUFB) + BI * LDB, s.head, s.t.kstart());
  };
  auto advance = [&](Step& s) {
    if (++s.jt >= total_tiles) {
      s.jt = 0;
      ++s.head;
      // re-read the item's first run rather than keep its seven words live in SGPRs
      const FFA_CONST int32_t* fr = itp + 8;
      asm volatile("" : "+s"(fr));
      tile_first(s.t, fr);
    } else {
      tile_next(s.t, rp, n_runs);
    }
  };

  float tsum = 0.0f;  // TOT: this lane's part of the current head's column sum
  auto write_total = [&](int head, float v) {
    if (row_ok && hh == 0) a.tot[(int64_t)b * a.t_sb + (int64_t)row * a.t_st + (int64_t)head * a.t_sh] = v;
  };
  // key-major: the tile's L (OL) or -Dd (OL + 1024) for the lane's 32 scores,
  // element e of the pair (xa, xb) in word e % 4 of read e / 4
  auto read_ld = [&](auto at_tag, f32x4_t(&w)[8]) {
    static_for<8>([&](auto i_tag) {
      constexpr int i = decltype(i_tag)::value;  // block i / 4, group i % 4
      w[i] = lds_read_b128<decltype(at_tag)::value + ((i >> 2) * 32 + (i & 3) * 8) * 4>(ld_addr);
    });
  };
  auto zero = [](f32x16_t& u, f32x16_t& w) {
#pragma unroll
    for (int i = 0; i < 16; ++i) { u[i] = 0.0f; w[i] = 0.0f; }
  };
  auto from = [](f32x4_t(&r)[8]) {
    return [&r](f32x16_t& u, f32x16_t& w) {
#pragma unroll
      for (int i = 0; i < 8; ++i) fence(r[i]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        u[e] = r[e >> 2][e & 3];
        w[e] = r[4 + (e >> 2)][e & 3];
      }
    };
  };
  // query-major step, or (TOT) a total-attention step: X1 and P only
  auto compute = [&](auto buf_tag, const Step& s) {
    constexpr int OA = decltype(buf_tag)::value * BUFB;
    constexpr int OB = OA + TILE;
    constexpr int OL = decltype(buf_tag)::value * LDB;  // relative to ld_addr
    f32x16_t xa, xb, ya, yb;
    // total attention, uncapped: X1 starts at -lse / scale; soft-capped, the lane
    // keeps lse * log2 e of its 32 queries (lv) for the tanh path
    f32x4_t lv[8];
    if constexpr (KV) read_ld(std::integral_constant<int, OL>{}, lv);
    if constexpr (KV && !CAP)
      rowprod(std::integral_constant<int, OA>{}, f1, xa, xb, [](auto) {}, from(lv));
    else
      rowprod(std::integral_constant<int, OA>{}, f1, xa, xb, [](auto) {}, zero);
    if constexpr (KV && CAP) {
      lds_wait<0>();
#pragma unroll
      for (int i = 0; i < 8; ++i) fence(lv[i]);
    }
    if (s.t.edge()) mask(s.t, xa, xb);
    if constexpr (TOT) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float x = e < 16 ? xa[e] : xb[e - 16];
        float arg;
        if constexpr (CAP) {
          const float th = tanh_from_2ylog2e(x * a.cap_arg);
          arg = x == -INFINITY ? -INFINITY : __builtin_fmaf(a.cap_log2, th, -lv[e >> 2][e & 3]);
        } else {
          arg = x * c2;
        }
        tsum += __builtin_amdgcn_exp2f(arg);
      }
      if (s.jt + 1 == total_tiles) {  // the head's last tile: its column sums are complete
        write_total(s.head, partner_sum(tsum));
        tsum = 0.0f;
      }
    } else {
      // query-major: P = exp2(X1 c2 - L) in place, between the MFMAs of X2.
      // Soft-capped: P = exp2(cap_log2 tanh - L) (masked scores stay at P = 0), and
      // what stays in place is P (1 - tanh^2), the factor of dS.
      constexpr int EPQ = 32 / (2 * KSTEPS);  // score elements per MFMA of X2
      V8 sf[4];
      rowprod(std::integral_constant<int, OB>{}, f2, ya, yb, [&](auto m_tag) {
        constexpr int m = decltype(m_tag)::value;
#pragma unroll
        for (int e = EPQ * m; e < EPQ * (m + 1); ++e) {
          if constexpr (CAP) {
            const float x = e < 16 ? xa[e] : xb[e - 16];
            const float th = tanh_from_2ylog2e(x * a.cap_arg);
            const float arg = x == -INFINITY ? -INFINITY : __builtin_fmaf(a.cap_log2, th, -l_row);
            const float pr = __builtin_amdgcn_exp2f(arg);
            const float keep = pr * __builtin_fmaf(-th, th, 1.0f);
            if (e < 16) xa[e] = keep;
            else xb[e - 16] = keep;
          } else {
            if (e < 16) xa[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(xa[e], c2, -l_row));
            else xb[e - 16] = __builtin_amdgcn_exp2f(__builtin_fmaf(xb[e - 16], c2, -l_row));
          }
        }
        fence(xa);
        fence(xb);
      }, zero);
      // dS = P (X2 - Dd) and its bf16 operand, one 16-row step t at a time: step
      // t + 1 behind the MFMAs of step t
      auto make_ds = [&](int t) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = 8 * t + u;
          const float p = e < 16 ? xa[e] : xb[e - 16];
          const float y = e < 16 ? ya[e] : yb[e - 16];
          sf[t][u] = (T)(p * (y + d_row));
        }
        fence(sf[t]);
      };
      make_ds(0);
      trprod(std::integral_constant<int, OA>{}, sf, acc1, [&](auto t_tag) {
        constexpr int t = decltype(t_tag)::value;
        if constexpr (t + 1 < 4) make_ds(t + 1);
      });
    }
  };

  // PAIR, role 0, step s in buffer BI: X1 (from -L), the edge mask, P = exp2(X1 c2)
  // -- soft-capped P = exp2(cap_log2 tanh - L) and the dS factor P (1 - tanh^2) --
  // handed over in bf16 at xa (the step's parity buffer), then dV += P^T dO.
  auto step_p = [&](auto buf_tag, const Step& s, uint32_t xa) {
    constexpr int BI = decltype(buf_tag)::value;
    f32x16_t pa, pb;
    f32x4_t lv[8];
    read_ld(std::integral_constant<int, BI * LDB>{}, lv);
    if constexpr (!CAP) {
      rowprod(std::integral_constant<int, BI * TILE>{}, f1, pa, pb, [](auto) {}, from(lv));
    } else {
      rowprod(std::integral_constant<int, BI * TILE>{}, f1, pa, pb, [](auto) {}, zero);
      lds_wait<0>();
#pragma unroll
      for (int i = 0; i < 8; ++i) fence(lv[i]);
    }
    if (s.t.edge()) mask(s.t, pa, pb);
    V8 pf[4], kf[4];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float x = e < 16 ? pa[e] : pb[e - 16];
      if constexpr (CAP) {
        const float th = tanh_from_2ylog2e(x * a.cap_arg);
        const float arg = x == -INFINITY ? -INFINITY : __builtin_fmaf(a.cap_log2, th, -lv[e >> 2][e & 3]);
        const float pr = __builtin_amdgcn_exp2f(arg);
        pf[e >> 3][e & 7] = (T)pr;
        kf[e >> 3][e & 7] = (T)(pr * __builtin_fmaf(-th, th, 1.0f));
      } else {
        pf[e >> 3][e & 7] = (T)__builtin_amdgcn_exp2f(x * c2);
      }
    }
    static_for<4>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      lds_write_b128<t * 1024>(xa, __builtin_bit_cast(f32x4_t, CAP ? kf[t] : pf[t]));
    });
    trprod(std::integral_constant<int, BI * TILE>{}, pf, acc1, [](auto) {});
  };
  // PAIR, role 1, the step before in buffer BI: X2 (from -Dd), then with the P its
  // partner handed over at xa one step earlier, dS = P (X2 - Dd) and dK += dS^T Q.
  auto step_ds = [&](auto buf_tag, uint32_t xa) {
    constexpr int BI = decltype(buf_tag)::value;
    f32x16_t ya, yb;
    f32x4_t dv[8];
    read_ld(std::integral_constant<int, BI * LDB + 1024>{}, dv);
    f32x4_t kr[4];
    rowprod(std::integral_constant<int, BI * TILE>{}, f1, ya, yb, [](auto) {}, from(dv));
    static_for<4>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      kr[t] = lds_read_b128<t * 1024>(xa);
    });
    lds_wait<0>();
#pragma unroll
    for (int t = 0; t < 4; ++t) fence(kr[t]);
    V8 sf[4];
    auto make_ds = [&](int t) {
      const V8 pk = as_v8<T>(kr[t]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = 8 * t + u;
        sf[t][u] = (T)((float)pk[u] * (e < 16 ? ya[e] : yb[e - 16]));
      }
      fence(sf[t]);
    };
    make_ds(0);
    trprod(std::integral_constant<int, BI * TILE>{}, sf, acc1, [&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      if constexpr (t + 1 < 4) make_ds(t + 1);
    });
  };

  if constexpr (PAIR) {
    // iteration j (0 .. steps): the tiles of step j + 1 are loaded, role 0 works on
    // step j, role 1 on step j - 1.  Step j's tiles sit in buffer j % 3 from
    // iteration j - 1 to iteration j + 1; its P in hand-over buffer j % 2 from
    // iteration j to j + 1.  The barrier at the top of each iteration orders every
    // reuse: buffer (j + 1) % 3 was last read by role 1 in iteration j - 1, hand-over
    // buffer j % 2 by role 1 in iteration j - 1 (and role 0's writes have landed).
    if (steps > 0) {
      Step cur;
      tile_first(cur.t, itp + 8);
      cur.head = hk * a.kv_ratio;
      cur.jt = 0;
      if (role == 1) load(std::integral_constant<int, 0>{}, cur);
      // top of iteration j: every wave's tiles of step j have landed (and role 0's
      // hand-over writes), then the DMA of step j + 1 into buffer (j + 1) % 3.
      // Returns step j + 1; cur stays step j for the work of the iteration.
      auto sync_load = [&](auto buf_tag, int j) {
        constexpr int P = decltype(buf_tag)::value;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_wait<0>();
        wg_barrier();
        Step nxt = cur;
        if (j + 1 < steps) {
          advance(nxt);
          if (role == 1) load(std::integral_constant<int, (P + 1) % 3>{}, nxt);
        }
        return nxt;
      };
      // The two roles run separate loops with the same barriers and DMAs, so that
      // neither carries the other's accumulator through a branch.
      if (role == 0) {
        auto it = [&](auto buf_tag, int j) {
          const Step nxt = sync_load(buf_tag, j);
          step_p(buf_tag, cur, x_addr + (uint32_t)((j & 1) * XB));
          cur = nxt;
        };
        int j = 0;
        for (; j + 3 <= steps; j += 3) {
          it(std::integral_constant<int, 0>{}, j);
          it(std::integral_constant<int, 1>{}, j + 1);
          it(std::integral_constant<int, 2>{}, j + 2);
        }
        if (j < steps) it(std::integral_constant<int, 0>{}, j);
        if (j + 1 < steps) it(std::integral_constant<int, 1>{}, j + 1);
        sync_load(std::integral_constant<int, 0>{}, steps);  // role 1's last step
      } else {
        cur = sync_load(std::integral_constant<int, 0>{}, 0);  // role 0's first step
        auto it = [&](auto buf_tag, int j) {
          constexpr int P = decltype(buf_tag)::value;
          cur = sync_load(buf_tag, j);
          // the dS / dK wave issues first when both waves of the SIMD are ready: its
          // VALU work is the lighter, so the exponentials of role 0 fill behind its
          // MFMAs rather than the other way round (measured: without the priority
          // -1 to -3.5%, with role 0 raised instead -5 to -7%)
          __builtin_amdgcn_s_setprio(1);
          step_ds(std::integral_constant<int, (P + 2) % 3>{}, x_addr + (uint32_t)(((j - 1) & 1) * XB));
          __builtin_amdgcn_s_setprio(0);
        };
        int j = 1;
        for (; j + 2 <= steps; j += 3) {
          it(std::integral_constant<int, 1>{}, j);
          it(std::integral_constant<int, 2>{}, j + 1);
          it(std::integral_constant<int, 0>{}, j + 2);
        }
        if (j <= steps) it(std::integral_constant<int, 1>{}, j);
        if (j + 1 <= steps) it(std::integral_constant<int, 2>{}, j + 1);
      }
    }
  } else if (steps > 0) {
    Step cur;
    tile_first(cur.t, itp + 8);
    cur.head = KV ? hk * a.kv_ratio : hq;
    cur.jt = 0;
    load(std::integral_constant<int, 0>{}, cur);
    auto iter = [&](auto buf_tag, int j) {
      constexpr int P = decltype(buf_tag)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      wg_barrier();
      Step nxt = cur;
      if (j + 1 < steps) {
        advance(nxt);
        load(std::integral_constant<int, 1 - P>{}, nxt);
      }
      compute(std::integral_constant<int, P>{}, cur);
      cur = nxt;
    };
    int j = 0;
    for (; j + 1 < steps; j += 2) {
      iter(std::integral_constant<int, 0>{}, j);
      iter(std::integral_constant<int, 1>{}, j + 1);
    }
    if (j < steps) iter(std::integral_constant<int, 0>{}, j);
  }

  if constexpr (TOT) {
    if (steps == 0)  // keys no query sees: total 0 for every head of the group
      for (int i = 0; i < heads_per_step; ++i) write_total(hk * a.kv_ratio + i, 0.0f);
    return;
  }
  // ---- epilogue: lane holds head-dim values 32 d + 8 gq + 4 hh + e of its row
  if (row_ok) {
    auto store = [&](__bf16* dst, const f32x16_t(&acc)[DBLK], float mul) {
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          if (32 * d + 8 * gq >= D) continue;  // D = 16: accumulator rows past the head dim
          V4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (T)(acc[d][4 * gq + e] * mul);
          *reinterpret_cast<V4*>(dst + 32 * d + 8 * gq + 4 * hh) = w;
        }
    };
    if constexpr (PAIR) {
      if (role) store(a.dk + (int64_t)b * a.dk_sb + (int64_t)row * a.dk_st + (int64_t)hk * a.dk_sh, acc1, a.scale);
      else store(a.dv + (int64_t)b * a.dv_sb + (int64_t)row * a.dv_st + (int64_t)hk * a.dv_sh, acc1, 1.0f);
    } else {
      store(a.dq + (int64_t)b * a.dq_sb + (int64_t)row * a.dq_st + (int64_t)hq * a.dq_sh, acc1, a.scale);
    }
  }
}

}  // namespace ffa::bwd

#ifndef FFA_BWD_KERNELS_ONLY
using namespace ffa::bwd;

// Compiled in ffa_bwd_small.hip: the instances for D = 16 and 32.
#define FFA_BWD_SMALL(D, T)                                                \
  extern template __global__ void ffa_bwd_main<D, false, false, false, T>(BwdArgs); \
  extern template __global__ void ffa_bwd_main<D, false, true, false, T>(BwdArgs);  \
  extern template __global__ void ffa_bwd_main<D, true, false, false, T>(BwdArgs);  \
  extern template __global__ void ffa_bwd_main<D, true, true, false, T>(BwdArgs);   \
  extern template __global__ void ffa_bwd_main<D, true, false, true, T>(BwdArgs);   \
  extern template __global__ void ffa_bwd_main<D, true, true, true, T>(BwdArgs);
namespace ffa::bwd {
FFA_BWD_SMALL(16, __bf16)
FFA_BWD_SMALL(16, _Float16)
FFA_BWD_SMALL(32, __bf16)
FFA_BWD_SMALL(32, _Float16)
}  // namespace ffa::bwd
#undef FFA_BWD_SMALL

static ffa_status hip_fail_b(hipError_t e, const char* what) {
  return ffa::set_error(FFA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" {

ffa_status ffa_total_attention(ffa_plan_t plan, const void* d_meta, int32_t batch, const void* q, int64_t q_sb,
                               int64_t q_st, int64_t q_sh, const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                               const float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh, float* total,
                               int64_t t_sb, int64_t t_st, int64_t t_sh, float softmax_scale,
                               const ffa_attn_extras* extras, void* d_workspace, size_t workspace_bytes,
                               void* stream) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  const ffa::Plan& p = plan->plan;
  if (p.bwd_off == 0)
    return ffa::set_error(FFA_ERR_ARG, "the plan has no key-major worklist (plan with FFA_PLAN_BACKWARD)");
  if (batch < 1) return ffa::set_error(FFA_ERR_ARG, "batch must be >= 1");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return ffa::set_error(FFA_ERR_ARG, "softmax_scale must be finite and > 0");
  if (!d_meta) return ffa::set_error(FFA_ERR_NULL, "d_meta is NULL");
  const bool has_q = p.total_q > 0, has_k = p.total_k > 0;
  const ffa_status xs = ffa::check_extras(extras, has_q);
  if (xs != FFA_OK) return xs;
  ffa_attn_extras ex = {};
  if (extras) ex = *extras;
  if (has_q && (!q || !lse)) return ffa::set_error(FFA_ERR_NULL, "q and lse must be non-NULL");
  if (has_k && (!k || !total)) return ffa::set_error(FFA_ERR_NULL, "k and total must be non-NULL");
  const int64_t ws_need = (int64_t)batch * p.bwd_workspace_bytes();
  if (ws_need > 0 && (!d_workspace || (int64_t)workspace_bytes < ws_need))
    return ffa::set_error(FFA_ERR_WORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                                 " bytes, total attention needs " + std::to_string(ws_need));
  auto al16 = [](const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; };
  auto st8 = [](int64_t x) { return (x & 7) == 0; };
  if ((has_q && !al16(q)) || (has_k && !al16(k)))
    return ffa::set_error(FFA_ERR_ALIGN, "q and k must be 16-byte aligned");
  for (int64_t x : {q_sb, q_st, q_sh, k_sb, k_st, k_sh})
    if (!st8(x)) return ffa::set_error(FFA_ERR_ALIGN, "q and k strides must be multiples of 8 elements");
  const int64_t lim = ((int64_t)1 << 31) / (2 * ffa::kBlockN);
  for (int64_t x : {k_st, q_st})
    if (x < 0 || x >= lim) return ffa::set_error(FFA_ERR_ARG, "q / k token strides must be in [0, 2^24) elements");
  if ((int64_t)p.num_kv_items * batch > INT32_MAX) return ffa::set_error(FFA_ERR_ARG, "grid too large");
  if ((int64_t)p.total_q * p.heads_q > ((int64_t)INT32_MAX) * 16) return ffa::set_error(FFA_ERR_ARG, "grid too large");

  hipStream_t s = (hipStream_t)stream;
  float* lw = static_cast<float*>(d_workspace);
  float* dwp = lw ? lw + (size_t)batch * p.heads_q * p.total_q : nullptr;
  if (has_q) {
    PreArgs pa = {};
    pa.lse = lse;
    pa.lw = lw;
    pa.dw = dwp;
    pa.l_sb = l_sb; pa.l_st = l_st; pa.l_sh = l_sh;
    pa.total_q = p.total_q;
    pa.heads_q = p.heads_q;
    pa.scale = softmax_scale;
    pa.fold = ex.softcap > 0.0f ? 0 : 1;
    const int ppb = 256 / (p.head_dim / 8);
    const int64_t pairs = (int64_t)p.total_q * p.heads_q;
    const dim3 grid((unsigned)((pairs + ppb - 1) / ppb), (unsigned)batch);
    dispatch_head_dim(p.head_dim, [&](auto d_tag) {
      dispatch_dtype(ex.dtype, [&](auto t_tag) {
        hipLaunchKernelGGL((ffa_bwd_pre<decltype(d_tag)::value, decltype(t_tag)>), grid, dim3(256), 0, s, pa);
      });
    });
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail_b(e, "launch ffa_bwd_pre");
  }
  if (p.num_kv_items == 0) return FFA_OK;
  const int32_t* bw = static_cast<const int32_t*>(d_meta) + p.bwd_off + ffa::kBwdHdr;
  const int32_t* kv_items = bw + (size_t)p.num_dq_items * kItemRec + (size_t)p.num_dq_runs * kRec;
  BwdArgs ba = {};
  ba.items = kv_items;
  ba.runs = kv_items + (size_t)p.num_kv_items * kItemRec;
  ba.q = static_cast<const __bf16*>(q);
  ba.k = static_cast<const __bf16*>(k);
  ba.q_sb = q_sb; ba.q_st = q_st; ba.q_sh = q_sh;
  ba.k_sb = k_sb; ba.k_st = k_st; ba.k_sh = k_sh;
  ba.lw = lw;
  ba.dw = dwp;
  ba.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  ba.scale = softmax_scale;
  ba.total_q = p.total_q;
  ba.total_k = p.total_k;
  ba.heads_q = p.heads_q;
  ba.batch = batch;
  ba.heads_per_item = p.heads_per_item;
  ba.kv_ratio = p.heads_q / p.heads_kv;
  const bool cap = ex.softcap > 0.0f;
  ba.cap_log2 = cap ? (float)((double)ex.softcap * 1.4426950408889634074) : 0.0f;
  ba.cap_arg = cap ? (float)(2.0 * 1.4426950408889634074 * (double)softmax_scale / (double)ex.softcap) : 0.0f;
  ba.tot = total;
  ba.t_sb = t_sb; ba.t_st = t_st; ba.t_sh = t_sh;
  const dim3 grid((unsigned)((int64_t)p.num_kv_items * batch));
  dispatch_head_dim(p.head_dim, [&](auto d_tag) {
    constexpr int D = decltype(d_tag)::value;
    dispatch_dtype(ex.dtype, [&](auto t_tag) {
      using T = decltype(t_tag);
      if (cap) hipLaunchKernelGGL((ffa_bwd_main<D, true, true, true, T>), grid, dim3(64 * ffa::kWaves), 0, s, ba);
      else hipLaunchKernelGGL((ffa_bwd_main<D, true, false, true, T>), grid, dim3(64 * ffa::kWaves), 0, s, ba);
    });
  });
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail_b(e, "launch ffa_bwd_main (total attention)");
  return FFA_OK;
}

ffa_status ffa_bwd(ffa_plan_t plan, const void* d_meta, int32_t batch, const void* q, int64_t q_sb, int64_t q_st,
                   int64_t q_sh, const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh, const void* v, int64_t v_sb,
                   int64_t v_st, int64_t v_sh, const void* out, int64_t o_sb, int64_t o_st, int64_t o_sh,
                   const float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh, const void* dout, int64_t d_sb,
                   int64_t d_st, int64_t d_sh, void* dq, int64_t dq_sb, int64_t dq_st, int64_t dq_sh, void* dk,
                   int64_t dk_sb, int64_t dk_st, int64_t dk_sh, void* dv, int64_t dv_sb, int64_t dv_st, int64_t dv_sh,
                   float softmax_scale, const ffa_attn_extras* extras, void* d_workspace, size_t workspace_bytes,
                   void* stream) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  const ffa::Plan& p = plan->plan;
  if (p.bwd_off == 0)
    return ffa::set_error(FFA_ERR_ARG, "the plan has no backward worklists (plan with FFA_PLAN_BACKWARD)");
  if (batch < 1) return ffa::set_error(FFA_ERR_ARG, "batch must be >= 1");
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return ffa::set_error(FFA_ERR_ARG, "softmax_scale must be finite and > 0");
  if (!d_meta) return ffa::set_error(FFA_ERR_NULL, "d_meta is NULL");
  const bool has_q = p.total_q > 0, has_k = p.total_k > 0;
  const ffa_status xs = ffa::check_extras(extras, has_q);
  if (xs != FFA_OK) return xs;
  ffa_attn_extras ex = {};
  if (extras) ex = *extras;
  if (has_q && (!q || !out || !lse || !dout || !dq))
    return ffa::set_error(FFA_ERR_NULL, "q, out, lse, dout and dq must be non-NULL");
  if (has_k && (!k || !v || !dk || !dv)) return ffa::set_error(FFA_ERR_NULL, "k, v, dk and dv must be non-NULL");
  const int64_t ws_need = (int64_t)batch * p.bwd_workspace_bytes();
  if (ws_need > 0 && (!d_workspace || (int64_t)workspace_bytes < ws_need))
    return ffa::set_error(FFA_ERR_WORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                                 " bytes, the backward needs " + std::to_string(ws_need));
  auto al16 = [](const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; };
  auto st8 = [](int64_t s) { return (s & 7) == 0; };
  if ((has_q && (!al16(q) || !al16(out) || !al16(dout) || !al16(dq))) ||
      (has_k && (!al16(k) || !al16(v) || !al16(dk) || !al16(dv))))
    return ffa::set_error(FFA_ERR_ALIGN, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  const int64_t sts[] = {q_sb, q_st, q_sh, k_sb, k_st, k_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh, d_sb, d_st, d_sh,
                         dq_sb, dq_st, dq_sh, dk_sb, dk_st, dk_sh, dv_sb, dv_st, dv_sh};
  for (int64_t x : sts)
    if (!st8(x)) return ffa::set_error(FFA_ERR_ALIGN, "bf16 tensor strides must be multiples of 8 elements");
  // the kernels address one 64-row tile with 32-bit offsets
  const int64_t lim = ((int64_t)1 << 31) / (2 * ffa::kBlockN);
  // (unsigned 32-bit offsets from the tile's first row: token strides must be >= 0)
  for (int64_t x : {k_st, v_st, q_st, d_st})
    if (x < 0 || x >= lim)
      return ffa::set_error(FFA_ERR_ARG, "q / k / v / dout token strides must be in [0, 2^24) elements");
  if (((int64_t)p.num_dq_items + p.num_kv_items) * batch > INT32_MAX) return ffa::set_error(FFA_ERR_ARG, "grid too large");
  if ((int64_t)p.total_q * p.heads_q > ((int64_t)INT32_MAX) * 16) return ffa::set_error(FFA_ERR_ARG, "grid too large");
  if (ex.n_sink > 0 && ex.dsink && has_q && (int64_t)ex.n_sink * p.heads_q > INT32_MAX)
    return ffa::set_error(FFA_ERR_ARG, "n_sink * heads_q too large");

  hipStream_t s = (hipStream_t)stream;
  float* lw = static_cast<float*>(d_workspace);
  float* dwp = lw ? lw + (size_t)batch * p.heads_q * p.total_q : nullptr;
  // L and -Dd of every (row, head) come from the query-major kernel, which runs
  // first: the key-major kernel and the sink gradient read them from the workspace.
  const int32_t* meta = static_cast<const int32_t*>(d_meta);
  const int32_t* bw = meta + p.bwd_off + ffa::kBwdHdr;
  const int32_t* dq_items = bw;
  const int32_t* dq_runs = dq_items + (size_t)p.num_dq_items * kItemRec;
  const int32_t* kv_items = dq_runs + (size_t)p.num_dq_runs * kRec;
  const int32_t* kv_runs = kv_items + (size_t)p.num_kv_items * kItemRec;

  BwdArgs ba = {};
  ba.q = static_cast<const __bf16*>(q);
  ba.k = static_cast<const __bf16*>(k);
  ba.v = static_cast<const __bf16*>(v);
  ba.dout = static_cast<const __bf16*>(dout);
  ba.dq = static_cast<__bf16*>(dq);
  ba.dk = static_cast<__bf16*>(dk);
  ba.dv = static_cast<__bf16*>(dv);
  ba.q_sb = q_sb; ba.q_st = q_st; ba.q_sh = q_sh;
  ba.k_sb = k_sb; ba.k_st = k_st; ba.k_sh = k_sh;
  ba.v_sb = v_sb; ba.v_st = v_st; ba.v_sh = v_sh;
  ba.d_sb = d_sb; ba.d_st = d_st; ba.d_sh = d_sh;
  ba.dq_sb = dq_sb; ba.dq_st = dq_st; ba.dq_sh = dq_sh;
  ba.dk_sb = dk_sb; ba.dk_st = dk_st; ba.dk_sh = dk_sh;
  ba.dv_sb = dv_sb; ba.dv_st = dv_st; ba.dv_sh = dv_sh;
  ba.lw = lw;
  ba.dw = dwp;
  ba.out = static_cast<const __bf16*>(out);
  ba.o_sb = o_sb; ba.o_st = o_st; ba.o_sh = o_sh;
  ba.lse = lse;
  ba.l_sb = l_sb; ba.l_st = l_st; ba.l_sh = l_sh;
  ba.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  ba.scale = softmax_scale;
  ba.total_q = p.total_q;
  ba.total_k = p.total_k;
  ba.heads_q = p.heads_q;
  ba.batch = batch;
  ba.heads_per_item = p.heads_per_item;
  ba.kv_ratio = p.heads_q / p.heads_kv;
  const bool cap = ex.softcap > 0.0f;
  ba.cap_log2 = cap ? (float)((double)ex.softcap * 1.4426950408889634074) : 0.0f;
  ba.cap_arg = cap ? (float)(2.0 * 1.4426950408889634074 * (double)softmax_scale / (double)ex.softcap) : 0.0f;

  const dim3 block(64 * ffa::kWaves);
  // the key-major kernel runs its pairs of waves: eight per workgroup
  const dim3 kv_block(64 * 2 * ffa::kWaves);
  if (p.num_dq_items > 0) {
    ba.items = dq_items;
    ba.runs = dq_runs;
    const dim3 grid((unsigned)((int64_t)p.num_dq_items * batch));
    dispatch_head_dim(p.head_dim, [&](auto d_tag) {
      constexpr int D = decltype(d_tag)::value;
      dispatch_dtype(ex.dtype, [&](auto t_tag) {
        using T = decltype(t_tag);
        if (cap) hipLaunchKernelGGL((ffa_bwd_main<D, false, true, false, T>), grid, block, 0, s, ba);
        else hipLaunchKernelGGL((ffa_bwd_main<D, false, false, false, T>), grid, block, 0, s, ba);
      });
    });
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail_b(e, "launch ffa_bwd_main (dq)");
  }
  if (p.num_kv_items > 0) {
    ba.items = kv_items;
    ba.runs = kv_runs;
    const dim3 grid((unsigned)((int64_t)p.num_kv_items * batch));
    dispatch_head_dim(p.head_dim, [&](auto d_tag) {
      constexpr int D = decltype(d_tag)::value;
      dispatch_dtype(ex.dtype, [&](auto t_tag) {
        using T = decltype(t_tag);
        static_assert(kBwdWgWaves<D, true, false> == 2 * ffa::kWaves, "block shape");
        if (cap) hipLaunchKernelGGL((ffa_bwd_main<D, true, true, false, T>), grid, kv_block, 0, s, ba);
        else hipLaunchKernelGGL((ffa_bwd_main<D, true, false, false, T>), grid, kv_block, 0, s, ba);
      });
    });
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail_b(e, "launch ffa_bwd_main (dk, dv)");
  }
  if (ex.n_sink > 0 && ex.dsink && has_q) {
    SinkArgs sa;
    sa.sink = ex.sink;
    sa.dsink = ex.dsink;
    sa.lw = lw;
    sa.dw = dwp;
    sa.sk_sb = ex.sink_sb; sa.sk_st = ex.sink_st; sa.sk_ss = ex.sink_ss; sa.sk_sh = ex.sink_sh;
    sa.total_q = p.total_q;
    sa.heads_q = p.heads_q;
    sa.n_sink = ex.n_sink;
    sa.l_mul = ex.softcap > 0.0f ? 1.0f : -ba.scale_log2;
    const dim3 grid((unsigned)((int64_t)ex.n_sink * p.heads_q), (unsigned)batch);
    hipLaunchKernelGGL(ffa_bwd_dsink, grid, dim3(256), 0, s, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail_b(e, "launch ffa_bwd_dsink");
  }
  return FFA_OK;
}

}  // extern "C"

#endif  // FFA_BWD_KERNELS_ONLY
