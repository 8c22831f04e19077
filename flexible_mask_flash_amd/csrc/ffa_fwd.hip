// gfx950 (MI355X) kernels and the C ABI of the flexible-mask attention forward.
//
// Main kernel (one workgroup = 4 wavefronts per plan item, two workgroups per CU):
//   * wavefront w covers 32 query rows of one query head; the workgroup covers
//     rows_per_item rows x heads_per_item heads that share one kv head, so a
//     K/V tile staged in LDS serves 128 (row, head) pairs.
//   * S^T = K Q^T per 64-key tile with v_mfma_f32_32x32x16_bf16: K is the A
//     operand (read from LDS), Q^T the B operand (held in registers for the
//     whole item).  Each lane then owns one query column and 16 keys per
//     32-key block, so the row max needs one cross-half exchange
//     (v_permlane32_swap) and the row sum stays per lane until the end.
//   * O^T += V^T P^T with the same MFMA: P^T comes straight from the S^T
//     registers (bf16), V^T from LDS with ds_read_b64_tr_b16 (4 keys of one
//     head-dim column per lane, two reads per MFMA operand).
//   * online softmax in fp32, base 2 (scale * log2 e folded into one FMA, done
//     for tile j+1 between the P V MFMAs of tile j).  A
//     row's reference point is the max of the first tile where it sees a key;
//     later tiles are exponentiated against it without a per-tile max, and
//     only when a probability would exceed 2^64 does the wave take the max,
//     rescale the accumulator and redo the tile (the result is the same: every
//     term of a row uses one reference point).
//   * K and V tiles are double-buffered in LDS and filled by
//     global_load_lds_dwordx4 (HBM -> LDS without registers), XOR-swizzled by
//     key row so that both the K row reads and the V transposed reads are
//     free of bank conflicts.
//   * causal / ragged edges are masked only on tiles past the item's n_full.
//   * out is divided by the row sum of the fp32 probabilities, or, with
//     FFA_EXTRAS_ROUNDED_NORM, by the sum of the 16-bit rounded ones that P V
//     multiplies (a second sum, 16 dot-product instructions per tile); lse
//     always comes from the fp32 sum.
//   * the epilogue writes bf16 out and fp32 lse, or -- for split items --
//     fp32 partial (out, lse) that ffa_combine merges with a global logsumexp
//     (FlagAttention user guide, "Split-KV and paged attention").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>

#include "ffa_device.h"

// Library-owned split-K workspace of ffa_fwd_noalloc (for callers that cannot
// allocate device memory): FFA_NOALLOC_SCRATCH_BYTES of device memory per GPU,
// held from the library's load until the process ends.  Host code never passes
// `scratch` itself to a kernel or a copy (its host-side name is not a device
// address); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[FFA_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace ffa::dev;
using ffa::kBlockN;
using ffa::kItemRec;
using ffa::kRec;
using ffa::kSlotsPerItem;

struct FwdArgs {
  const int32_t* items;
  const int32_t* runs;
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* out;
  float* lse;
  int64_t q_sb, q_st, q_sh;
  int64_t k_sb, k_st, k_sh;
  int64_t v_sb, v_st, v_sh;
  int64_t o_sb, o_st, o_sh;
  int64_t l_sb, l_st, l_sh;
  float* ws_o;       // [batch][slots][D]
  float* ws_lse;     // [batch][slots]
  int64_t ws_slots;  // slots per batch element
  float scale_log2;  // softmax_scale * log2(e)
  int32_t total_k;
  int32_t batch;
  int32_t heads_per_item;
  int32_t kv_ratio;  // heads_q / heads_kv
  // soft-capping (CAP instances): score -> softcap * tanh(scale q.k / softcap)
  float cap_log2;    // softcap * log2(e)
  float cap_arg;     // 2 * log2(e) * scale / softcap: tanh(y) = 1 - 2 / (1 + exp2(cap_arg * q.k))
  // attention sink: n_sink logits per (row, head) at sink[b*sk_sb + row*sk_st + s*sk_ss + h*sk_sh]
  const float* sink;
  int64_t sk_sb, sk_st, sk_ss, sk_sh;
  int32_t n_sink;
};

struct CombineArgs {
  const int32_t* combine;
  const float* ws_o;
  const float* ws_lse;
  int64_t ws_slots;
  __bf16* out;
  float* lse;
  int64_t o_sb, o_st, o_sh;
  int64_t l_sb, l_st, l_sh;
  int32_t batch;
  int32_t heads_per_item;
  const float* sink;
  int64_t sk_sb, sk_st, sk_ss, sk_sh;
  int32_t n_sink;
};

// tanh(y) with y given as 2 y log2(e): 1 - 2 / (1 + 2^(2 y log2 e)); exact limits
// +-1 for +-inf, absolute error ~1e-7 near 0 (fp32 rounding of 1)
__device__ __forceinline__ float tanh_from_2ylog2e(float z) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// A row keeps its reference point (log2 units) until one of its probabilities
// would exceed ElemT<T>::kMaxP (2^64 for bf16, 2^15 for fp16, whose largest value
// is 65504): a lane's per-tile partial sum above it sends the whole wave through
// the exact rescale path.  Values up to that bound are exact enough in the
// element type and fp32 (relative rounding) and cannot overflow the fp32 sums.

// LDS row swizzles (16-byte chunk index XOR by key row).
//  K rows are read as MFMA A operands: lanes 0-15 read one chunk of rows
//  r..r+15, so the XOR spreads those 16 rows over all 16-byte bank groups.
//  V rows are read transposed: a 16-lane group reads two chunks of four
//  consecutive rows, so four consecutive rows are spread by 4 chunks.
//  At D = 32 a row is 64 bytes, so four consecutive rows already fill one
//  256-byte bank window: the transposed V reads need no swizzle, and the K rows
//  r .. r+15 only need the XOR by their window index.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : D == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 3) << 2) : D == 64 ? (((r >> 1) & 1) << 2) : 0;
}

// c + a.x + a.y of a 16-bit pair (one dot-product instruction against (1, 1))
template <typename T>
__device__ __forceinline__ float dot2_ones(typename ElemT<T>::v2 a, float c) {
  const typename ElemT<T>::v2 ones = {(T)1.0f, (T)1.0f};
  if constexpr (std::is_same<T, _Float16>::value)
    return __builtin_amdgcn_fdot2(a, ones, c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(a, ones, c, false);
}

// Waves per SIMD the compiler budgets registers for: two at D = 128 (256 VGPRs), more
// below, where O and the fragments shrink but the per-score softmax work does not, so a
// third or fourth wave hides more of it (+4.5% at D = 64 with three, +4 to +6% at
// D = 32 and 16 with four; the few spills this costs sit outside the tile loop).
template <int D>
constexpr int kFwdWaves = D <= 32 ? 4 : D <= 64 ? 3 : 2;

// RN: out is divided by the sum of the 16-bit rounded weights that P V multiplies
// (lse keeps the sum of the fp32 weights), so the output is a convex combination of
// value rows up to fp32 accumulation (FFA_EXTRAS_ROUNDED_NORM).
template <int D, bool CAP, bool RN, typename T>
__global__ __launch_bounds__(64 * ffa::kWaves) __attribute__((amdgpu_waves_per_eu(kFwdWaves<D>, kFwdWaves<D>))) void ffa_fwd_main(FwdArgs a) {
  using V8 = typename ElemT<T>::v8;
  using V4 = typename ElemT<T>::v4;
  using V2 = typename ElemT<T>::v2;
  (void)sizeof(V2);
  constexpr int BN = kBlockN;          // 64 keys per tile
  // D = 16 keeps its K and V tiles in the 32-wide layout: one MFMA k-step covers
  // the 16 head dims of a score, and the unused half of a V row only feeds rows
  // 16-31 of the O accumulator, which are never stored (so the DMA may leave
  // anything there, as long as it reads nothing outside the tensors).
  constexpr int DL = D < 32 ? 32 : D;  // head dims of an LDS row and of O
  constexpr int GC = D / 8;            // 16-byte chunks of a global row
  constexpr int ROWB = DL * 2;         // bytes of one K/V row in LDS
  constexpr int CH = DL / 8;           // 16-byte chunks per LDS row
  constexpr int KSTEPS = D / 16;       // MFMA k-steps of K Q^T per 32-key block
  constexpr int DBLK = DL / 32;        // 32-wide head-dim blocks of O
  constexpr int TILE = BN * ROWB;      // bytes of one K or V tile
  constexpr int W = ffa::kWaves;       // wavefronts sharing the DMA of a tile
  constexpr int NLD = TILE / (1024 * W);  // DMA instructions per thread per K (or V) tile
  constexpr int RPL = 1024 * W / ROWB;    // key rows between consecutive DMA instructions
  static_assert(NLD * 1024 * W == TILE, "DMA split");
  constexpr int QSLOTS = 2 * KSTEPS;   // MFMAs of one K Q^T tile
  constexpr int EPQ = 32 / QSLOTS;     // score elements exponentiated per K Q^T MFMA
  static_assert(BN == 64 && (D == 16 || D == 32 || D == 64 || D == 128), "tile shape");
  // one LDS array: K0 | V0 | K1 | V1; every read offset is a compile-time immediate
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  constexpr int kOffK[2] = {0, 2 * TILE};
  constexpr int kOffV[2] = {TILE, 3 * TILE};

  // The first tile waits on a chain of dependent loads: arguments -> item record
  // -> Q and the first K/V tile.  Each fence below makes its whole group of
  // scalar loads issue together (the compiler would otherwise sink every load
  // next to its first use, one more round trip each).
  asm volatile("" ::"s"(a.items), "s"(a.runs), "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.q_sb), "s"(a.q_st),
               "s"(a.q_sh), "s"(a.k_sb), "s"(a.k_st), "s"(a.k_sh), "s"(a.v_sb), "s"(a.v_st), "s"(a.v_sh),
               "s"(a.total_k), "s"(a.batch), "s"(a.heads_per_item), "s"(a.kv_ratio));
  const int bid = blockIdx.x;
  const int item_idx = bid / a.batch;
  const int b = bid - item_idx * a.batch;
  const FFA_CONST int32_t* itp = (const FFA_CONST int32_t*)(a.items + (int64_t)item_idx * kItemRec);
  const int q0 = itp[0], nrows = itp[1], h0 = itp[2], run_off = itp[3], n_runs = itp[4];
  const int slot = itp[5], total_tiles = itp[6];
  asm volatile("" ::"s"(q0), "s"(nrows), "s"(h0), "s"(run_off), "s"(n_runs), "s"(slot), "s"(total_tiles),
               "s"(itp[8]), "s"(itp[9]), "s"(itp[10]), "s"(itp[11]), "s"(itp[12]));

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hh = lane >> 5;            // which half of the 64 lanes
  const int G = a.heads_per_item;
  const int g = wave % G, rsub = wave / G;
  const int h = h0 + g;
  const int hk = h0 / a.kv_ratio;
  const int lrow = rsub * 32 + (lane & 31);
  const int row = q0 + lrow;
  const bool row_ok = lrow < nrows;

  const char* kbase = (const char*)(a.k + (int64_t)b * a.k_sb + (int64_t)hk * a.k_sh);
  const char* vbase = (const char*)(a.v + (int64_t)b * a.v_sb + (int64_t)hk * a.v_sh);

  // ---- Q^T operand: lane holds query `row`, head-dim half hh (D/2 contiguous values)
  V8 qf[KSTEPS];
  if (row_ok && n_runs > 0) {
    const V8* qp = reinterpret_cast<const V8*>(a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh +
                                                           (int64_t)row * a.q_st + hh * (D / 2));
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = qp[s];
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[s][j] = (T)0.0f;
  }

  f32x16_t o[DBLK];
#pragma unroll
  for (int d = 0; d < DBLK; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.0f;
  float m_run = -INFINITY;  // running max, log2 units (already scaled)
  float l_run = 0.0f;       // this lane's part of the row sum
  float lr_run = 0.0f;      // RN: the same sum of the rounded weights

  // ---- per-lane LDS read addresses (the low 10 bits of the LDS base are zero)
  const uint32_t lds = (uint32_t)(uintptr_t)(FFA_LDS char*)smem;
  // K fragment of k-step s: row (lane & 31) (+32 per key block), chunk (D/16)*hh + s
  uint32_t k_addr[KSTEPS];
  {
    const int r = lane & 31;
    const uint32_t a0 = lds + r * ROWB + ((((D / 16) * hh) ^ swz_k<DL>(r)) << 4);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) k_addr[s] = a0 ^ (s << 4);
  }
  // V^T fragment of head-dim block d: rows 4hh + j/4 (+16 t, +8), column 32d + 16(grp&1) + 4(j&3)
  uint32_t v_addr[DBLK];
  {
    const int grp = lane >> 4, jl = lane & 15;
    const int vr = 4 * hh + (jl >> 2);
    const int cl = 2 * (grp & 1) + ((jl & 3) >> 1);
    const uint32_t a0 = lds + vr * ROWB + ((cl ^ swz_v<DL>(vr)) << 4) + (jl & 1) * 8;
#pragma unroll
    for (int d = 0; d < DBLK; ++d) v_addr[d] = a0 ^ (d << 6);
  }

  // ---- DMA of a K or V tile: instruction i of wave w fills LDS block (W i + w) of
  // the tile; lane l's 16 bytes are chunk (lin % CH) of key row (lin / CH),
  // lin = 64 (W i + w) + l, loaded from the swizzled global chunk.  The lane's
  // offset is the same for every i up to whole rows, so each load is a scalar
  // base plus one constant 32-bit per-lane offset.
  const int lin0 = wave * 64 + lane;
  const int dr0 = lin0 / CH, dp = lin0 % CH;
  const int64_t kst_b = a.k_st * 2, vst_b = a.v_st * 2;
  uint32_t k_goff = (uint32_t)(dr0 * kst_b) + ((dp ^ swz_k<DL>(dr0)) << 4);
  uint32_t v_goff = (uint32_t)(dr0 * vst_b) + ((dp ^ swz_v<DL>(dr0)) << 4);
  if constexpr (GC < CH) {
    // padding lanes of a D = 16 row: an offset past the buffer's end loads zeros
    // without touching memory
    if ((dp ^ swz_k<DL>(dr0)) >= GC) k_goff = 0x80000000u;
    if ((dp ^ swz_v<DL>(dr0)) >= GC) v_goff = 0x80000000u;
  }
  auto dma = [&](const char* base, int64_t st_b, uint32_t goff, int swzc, char* dst, int kstart) {
    if (kstart + BN <= a.total_k) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kstart * st_b), (short)0, 0x7fffffff, kBufferFlags);
      // LDS destinations and row offsets are recomputed here with scalar adds;
      // hoisted out of the tile loop they would be 2 x NLD long-lived scalars
      // per tensor and buffer, spilled to VGPR lanes and read back by the VALU.
      uint32_t ldst = (uint32_t)(uintptr_t)(FFA_LDS char*)dst + wave * 1024;
      int32_t rstep = (int32_t)(RPL * st_b);
      asm volatile("" : "+s"(ldst), "+s"(rstep));
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FFA_LDS void*)(uintptr_t)(ldst + i * W * 1024), 16, goff,
                                                 i * rstep, 0, 0);
    } else {
      // last tile of the key axis: rows past total_k re-read the last row (they are masked).
      // The empty asm keeps this path's per-lane address arithmetic inside the branch
      // (hoisted above it, it would run on every tile).
      asm volatile("" : "+s"(kstart));
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int key = min(kstart + dr0 + i * RPL, a.total_k - 1);
        int lc = dp ^ swzc;
        if constexpr (GC < CH) lc = lc < GC ? lc : 0;  // padding lanes re-read chunk 0 of the row
        __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)key * st_b + (lc << 4)),
                                         (FFA_LDS void*)(dst + (i * W + wave) * 1024), 16, 0, 0);
      }
    }
  };
  auto dma_k = [&](auto buf_tag, int kstart) {
    constexpr int BUF = decltype(buf_tag)::value;
    dma(kbase, kst_b, k_goff, swz_k<DL>(dr0), smem + kOffK[BUF], kstart);
  };
  auto dma_v = [&](auto buf_tag, int kstart) {
    constexpr int BUF = decltype(buf_tag)::value;
    dma(vbase, vst_b, v_goff, swz_v<DL>(dr0), smem + kOffV[BUF], kstart);
  };

  // ---- K Q^T of one tile from K buffer BUF into (sa, sb); hook(slot) runs after
  // the slot-th MFMA is issued, so independent VALU work overlaps the MFMAs
  auto qk = [&](auto buf_tag, f32x16_t& sa, f32x16_t& sb, auto&& hook) {
    constexpr int OK = kOffK[decltype(buf_tag)::value];
    constexpr int NQ = 2 * KSTEPS;   // fragments of the tile, in MFMA order
    constexpr int KIF = NQ < 4 ? NQ : 4;  // fragment reads in flight (a ring of KIF registers)
    // MFMA m uses k-step m/2 of key block m%2: the two accumulator chains
    // alternate, so consecutive MFMAs never depend on each other
#pragma unroll
    for (int i = 0; i < 16; ++i) { sa[i] = 0.0f; sb[i] = 0.0f; }
    __builtin_amdgcn_s_setprio(1);
    f32x4_t kf[KIF];
    static_for<KIF>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      kf[m] = lds_read_b128<OK + (m % 2) * 32 * ROWB>(k_addr[m / 2]);
    });
    static_for<NQ>([&](auto m_tag) {
      constexpr int m = decltype(m_tag)::value;
      constexpr int later = (m + KIF - 1 < NQ - 1) ? KIF - 1 : NQ - 1 - m;  // reads issued after read m
      lds_wait<later>();
      fence(kf[m % KIF]);
      if constexpr (m % 2 == 0)
        sa = mfma32(as_v8<T>(kf[m % KIF]), qf[m / 2], sa);
      else
        sb = mfma32(as_v8<T>(kf[m % KIF]), qf[m / 2], sb);
      if constexpr (m + KIF < NQ) {
        constexpr int r = m + KIF;
        kf[m % KIF] = lds_read_b128<OK + (r % 2) * 32 * ROWB>(k_addr[r / 2]);
      }
      hook(std::integral_constant<int, m>{});
    });
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- O^T += V^T P^T of one tile from V buffer BUF (16 keys per MFMA; the reads
  // of step t+1 are in flight during the MFMAs of step t); hook(slot) as above
  auto pv = [&](auto buf_tag, const V8 (&pf)[4], auto&& hook) {
    constexpr int OV = kOffV[decltype(buf_tag)::value];
    s16x4_t vlo[2][DBLK], vhi[2][DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d) {
      vlo[0][d] = lds_read_tr16<OV>(v_addr[d]);
      vhi[0][d] = lds_read_tr16<OV + 8 * ROWB>(v_addr[d]);
    }
    static_for<4>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      constexpr int cur = t & 1, nxt = cur ^ 1;
      if constexpr (t + 1 < 4) {
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
          vlo[nxt][d] = lds_read_tr16<OV + 16 * (t + 1) * ROWB>(v_addr[d]);
          vhi[nxt][d] = lds_read_tr16<OV + (16 * (t + 1) + 8) * ROWB>(v_addr[d]);
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
        o[d] = mfma32(__builtin_bit_cast(V8, vv), pf[t], o[d]);
        hook(std::integral_constant<int, t * DBLK + d>{});
      });
    });
  };

  // edge mask of a tile's scores: key j (absolute) visible iff
  // row + lo_base <= j < min(k_hi, row + edge_base); the lower bound only exists
  // for slices whose start moves with the row (inverse causal, bi-causal)
  auto mask = [&](const TileIt& t, f32x16_t& sa, f32x16_t& sb) {
    const int base = t.kstart() + 4 * hh;
    const int lim = min(t.khi, row + t.eb) - base;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rel = 8 * (i >> 2) + (i & 3);
      if (rel >= lim) sa[i] = -INFINITY;
      if (rel + 32 >= lim) sb[i] = -INFINITY;
    }
    if (t.lb != -ffa::kNoEdge) {
      const int low = row + t.lb - base;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rel = 8 * (i >> 2) + (i & 3);
        if (rel < low) sa[i] = -INFINITY;
        if (rel + 32 < low) sb[i] = -INFINITY;
      }
    }
  };

  const float c2 = a.scale_log2;
  const float cap_arg = a.cap_arg;
  const FFA_CONST int32_t* rp = (const FFA_CONST int32_t*)(a.runs + (int64_t)run_off * kRec);

  if (total_tiles > 0) {
    // Software pipeline: iteration j exponentiates the scores of tile j while the
    // MFMAs of K Q^T for tile j+1 run, then multiplies P_j V_j while the scores of
    // tile j+1 are masked and max-reduced.  K is one tile ahead of V:
    // LDS holds K_{j+1}, V_j, and receives K_{j+2}, V_{j+1} during iteration j.
    TileIt t0;
    tile_first(t0, itp + 8);  // the inline copy of runs[run_off]
    dma_k(std::integral_constant<int, 0>{}, t0.kstart());
    dma_v(std::integral_constant<int, 0>{}, t0.kstart());
    TileIt tA = t0, tB;   // tA: tile j+1, tB: tile j+2
    tile_next(tA, rp, n_runs);
    tB = tA;
    tile_next(tB, rp, n_runs);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    wg_barrier();
    if (total_tiles > 1) dma_k(std::integral_constant<int, 1>{}, tA.kstart());

    // two score sets alternate between even and odd tiles (no copies)
    f32x16_t sa0, sb0, sa1, sb1;
    qk(std::integral_constant<int, 0>{}, sa0, sb0, [](auto) {});
    if (t0.edge()) mask(t0, sa0, sb0);

    // Reference point and exponent arguments of a tile, computed in place
    // (x = s * c2 - m) one tile ahead of its exponentials.  A row that has not
    // met a visible key yet (m_run = -inf) takes the max of this tile; every
    // other row keeps its reference, and the overflow check after the
    // exponentials restores the exact max when a tile's scores outgrow it by
    // more than 2^64.  msub_next is the reference the arguments were taken with.
    float msub_next = 0.0f;
    // soft-capped argument of a raw score (masked scores stay -inf)
    auto capped = [&](float x) -> float {
      const float th = tanh_from_2ylog2e(x * cap_arg);
      return x == -INFINITY ? -INFINITY : a.cap_log2 * th;
    };
    auto reference = [&](f32x16_t& xa, f32x16_t& xb) {
      if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY)) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(fmaxf(mx, xa[i]), xb[i]);
        mx = partner_max(mx);
        if (m_run == -INFINITY) m_run = CAP ? capped(mx) : mx * c2;
      }
      msub_next = (m_run == -INFINITY) ? 0.0f : m_run;
    };
    auto prep = [&](f32x16_t& xa, f32x16_t& xb, int e0, int e1) {
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        if constexpr (CAP) {
          if (e < 16) xa[e] = capped(xa[e]) - msub_next;
          else xb[e - 16] = capped(xb[e - 16]) - msub_next;
        } else {
          if (e < 16) xa[e] = __builtin_fmaf(xa[e], c2, -msub_next);
          else xb[e - 16] = __builtin_fmaf(xb[e - 16], c2, -msub_next);
        }
      }
    };
    reference(sa0, sb0);
    prep(sa0, sb0, 0, 32);

    auto iter = [&](auto buf_tag, auto next_tag, int j, f32x16_t& ca, f32x16_t& cb, f32x16_t& na,
                    f32x16_t& nb) {
      constexpr int P = decltype(buf_tag)::value;  // V_j in V buffer P, K_{j+1} in K buffer 1-P
      constexpr bool NEXT = decltype(next_tag)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      wg_barrier();
      if constexpr (NEXT) {
        if (j + 2 < total_tiles) dma_k(std::integral_constant<int, P>{}, tB.kstart());
        dma_v(std::integral_constant<int, 1 - P>{}, tA.kstart());
      }

      const float msub = msub_next;  // reference of tile j's arguments

      // P_j = exp2(x_j), interleaved with K Q^T of tile j+1 (the arguments x_j were
      // prepared during the previous P V).  Each hook packs its probabilities into
      // bf16 pairs and pins them (and the running sum) with fence(), so the work
      // stays between the MFMAs it is meant to overlap instead of sinking to its
      // use in P V.
      uint32_t pu[16];  // bf16 pairs of P_j, pair q = elements 2q, 2q+1
      float ps = 0.0f;
      auto exp_hook = [&](auto slot_tag) {
        constexpr int sl = decltype(slot_tag)::value;
#pragma unroll
        for (int e = sl * EPQ; e < (sl + 1) * EPQ; e += 2) {
          const float s0v = e < 16 ? ca[e] : cb[e - 16];
          const float s1v = e + 1 < 16 ? ca[e + 1] : cb[e + 1 - 16];
          const float p0 = __builtin_amdgcn_exp2f(s0v);
          const float p1 = __builtin_amdgcn_exp2f(s1v);
          ps = e == 0 ? p0 + p1 : ps + (p0 + p1);  // no 0 + x add for the first pair
          const V2 pr = {(T)p0, (T)p1};
          pu[e >> 1] = __builtin_bit_cast(uint32_t, pr);
          fence(pu[e >> 1]);
        }
        fence(ps);
      };
      if constexpr (NEXT) {
        qk(std::integral_constant<int, 1 - P>{}, na, nb, exp_hook);
      } else {
        static_for<QSLOTS>(exp_hook);
      }
      if (__builtin_amdgcn_ballot_w64(!(ps <= ElemT<T>::kMaxP))) {
        // rare: some probability above 2^64 -- move the reference to the row max
        // of this tile, rescale what is accumulated, and redo the tile (the
        // arguments hold s * c2 - msub)
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(fmaxf(mx, ca[i]), cb[i]);
        mx = partner_max(mx);
        const float m_new = fmaxf(m_run, mx + msub);
        const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = m_new;
        l_run *= alpha;
        if constexpr (RN) lr_run *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
        const float shift = (m_run == -INFINITY) ? 0.0f : m_run - msub;
        ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f((e < 16 ? ca[e] : cb[e - 16]) - shift);
          const float p1 = __builtin_amdgcn_exp2f((e + 1 < 16 ? ca[e + 1] : cb[e + 1 - 16]) - shift);
          ps += p0 + p1;
                    const V2 pr = {(T)p0, (T)p1};
          pu[e >> 1] = __builtin_bit_cast(uint32_t, pr);
        }
      }
      l_run += ps;
      // RN: the sum of the rounded weights, formed between the P V MFMAs (the K Q^T
      // section's VALU slots are taken by the exponentials)
      float pr_s = 0.0f;
      auto rs_hook = [&](auto slot_tag) {
        if constexpr (RN) {
          constexpr int sl = decltype(slot_tag)::value;
          constexpr int PPS = 16 / (4 * DBLK);
#pragma unroll
          for (int q = sl * PPS; q < (sl + 1) * PPS; ++q)
            pr_s = dot2_ones<T>(__builtin_bit_cast(V2, pu[q]), pr_s);
          fence(pr_s);
        }
      };
      V8 pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t w = {pu[4 * t], pu[4 * t + 1], pu[4 * t + 2], pu[4 * t + 3]};
        pf[t] = __builtin_bit_cast(V8, w);
      }

      // O += P_j V_j; the edge mask and reference point of tile j+1 go first, its
      // exponent arguments are prepared between the MFMAs (this keeps the FMAs
      // out of the K Q^T section, where the exponentials already take the VALU)
      if constexpr (NEXT) {
        if (tA.edge()) mask(tA, na, nb);
        reference(na, nb);
        pv(std::integral_constant<int, P>{}, pf, [&](auto slot_tag) {
          constexpr int sl = decltype(slot_tag)::value;
          constexpr int EPP = 32 / (4 * DBLK);
          prep(na, nb, sl * EPP, (sl + 1) * EPP);
          fence(na);
          fence(nb);
          rs_hook(slot_tag);
        });
        tA = tB;
        tile_next(tB, rp, n_runs);
      } else {
        pv(std::integral_constant<int, P>{}, pf, rs_hook);
      }
      if constexpr (RN) lr_run += pr_s;
    };

    // steady state: pairs of iterations that both have a next tile
    int j = 0;
    for (; j + 2 < total_tiles; j += 2) {
      iter(std::integral_constant<int, 0>{}, std::true_type{}, j, sa0, sb0, sa1, sb1);
      iter(std::integral_constant<int, 1>{}, std::true_type{}, j + 1, sa1, sb1, sa0, sb0);
    }
    // tail: one or two tiles left, the last one without a successor
    if (j + 1 < total_tiles) {
      iter(std::integral_constant<int, 0>{}, std::true_type{}, j, sa0, sb0, sa1, sb1);
      iter(std::integral_constant<int, 1>{}, std::false_type{}, j + 1, sa1, sb1, sa0, sb0);
    } else {
      iter(std::integral_constant<int, 0>{}, std::false_type{}, j, sa0, sb0, sa1, sb1);
    }
  }

  // ---- epilogue
  // The output pointers and strides are read again from the argument segment
  // through a pointer the compiler cannot see through, so that they are not
  // held in scalar registers (or spilled) across the tile loop.
  const FFA_CONST FwdArgs* ea = (const FFA_CONST FwdArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ea));
  const float lsum = partner_sum(l_run);
  const float lnorm = RN ? partner_sum(lr_run) : lsum;  // what out is divided by
  float inv = lsum > 0.0f ? 1.0f / lnorm : 0.0f;
  float lse_v = lsum > 0.0f ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
  const int n_sink = ea->n_sink;
  if (n_sink > 0 && slot < 0 && row_ok) {
    // sink logits join the denominator (split rows get them in the combine)
    const float* sp = ea->sink + (int64_t)b * ea->sk_sb + (int64_t)row * ea->sk_st + (int64_t)h * ea->sk_sh;
    const int64_t ss = ea->sk_ss;
    float ms = -INFINITY;
    for (int s = 0; s < n_sink; ++s) ms = fmaxf(ms, sp[s * ss] * kLog2e);
    const float mk = lsum > 0.0f ? m_run : -INFINITY;
    const float mt = fmaxf(mk, ms);
    if (mt != -INFINITY) {
      const float fk = __builtin_amdgcn_exp2f(mk - mt);  // 0 when the row sees no key
      float lt = lsum * fk, ln = lnorm * fk;
      for (int s = 0; s < n_sink; ++s) {
        const float e = __builtin_amdgcn_exp2f(sp[s * ss] * kLog2e - mt);
        lt += e;
        if constexpr (RN) ln += e;
      }
      inv = fk / (RN ? ln : lt);
      lse_v = (mt + __log2f(lt)) * kLn2;
    }
  }
  if (slot < 0) {
    // all the output arguments in one round trip (each use would otherwise
    // reload its own field right before its store)
    __bf16* const out_p = ea->out;
    float* const lse_p = ea->lse;
    const int64_t o_sb = ea->o_sb, o_st = ea->o_st, o_sh = ea->o_sh;
    const int64_t l_sb = ea->l_sb, l_st = ea->l_st, l_sh = ea->l_sh;
    asm volatile("" ::"s"(out_p), "s"(lse_p), "s"(o_sb), "s"(o_st), "s"(o_sh), "s"(l_sb), "s"(l_st), "s"(l_sh));
    // Stage the bf16 tile of this wave (32 rows x D) in LDS, then write whole
    // rows with 16-byte stores: in the MFMA layout a lane holds 4 consecutive
    // values of each of 16 head-dim groups, which would otherwise become 8-byte
    // stores spread over 32 rows.  Every wave is past its last LDS read first.
    // out and lse are written once and not read again by this launch: stored
    // non-temporal (measured: the workgroup's end, which waits for its stores,
    // comes earlier).
    wg_barrier();
    char* st = smem + wave * (32 * ROWB);
    {
      const int q = lane & 31;
#pragma unroll
      for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          V4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (T)(o[d][4 * gq + e] * inv);
          const int c = 4 * d + gq;  // 16-byte chunk of the row
          *reinterpret_cast<V4*>(st + q * ROWB + ((c ^ swz_k<DL>(q)) << 4) + hh * 8) = w;
        }
    }
    __bf16* ob = out_p + (int64_t)b * o_sb + (int64_t)h * o_sh;
    const int r0 = q0 + rsub * 32;
    const int nvalid = min(32, nrows - rsub * 32);
    constexpr int NST = 32 * CH / 64;  // 16-byte chunks per lane
    f32x4_t val[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {  // every read issued before the first store
      const int lin = i * 64 + lane;
      const int r = lin / CH, c = lin % CH;
      val[i] = *reinterpret_cast<const f32x4_t*>(st + r * ROWB + ((c ^ swz_k<DL>(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int lin = i * 64 + lane;
      const int r = lin / CH, c = lin % CH;
      if (r < nvalid && c < GC)
        __builtin_nontemporal_store(val[i], reinterpret_cast<f32x4_t*>(ob + (int64_t)(r0 + r) * o_st + c * 8));
    }
    if (row_ok && hh == 0)
      __builtin_nontemporal_store(lse_v, lse_p + (int64_t)b * l_sb + (int64_t)row * l_st + (int64_t)h * l_sh);
  } else if (row_ok) {
    const int64_t sidx = (int64_t)b * ea->ws_slots + slot + lrow * G + g;
    float* op = ea->ws_o + sidx * D;
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        if (32 * d + 8 * gq >= D) continue;  // D = 16: the O rows past the head dim
        f32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[d][4 * gq + e] * inv;
        *reinterpret_cast<f32x4_t*>(op + 32 * d + 8 * gq + 4 * hh) = w;
      }
    if (hh == 0) ea->ws_lse[sidx] = lse_v;
  }
}

// Merge split partials: lse = ln sum_c exp(lse_c); out = sum_c exp(lse_c - lse) out_c.
// One workgroup per combine entry (up to 128 (row, head) pairs); D/4 lanes per pair.
template <int D, typename T>
__global__ __launch_bounds__(256) void ffa_combine(CombineArgs a) {
  using V4 = typename ElemT<T>::v4;
  constexpr int TPP = D / 4;          // threads per (row, head) pair
  constexpr int PPP = 256 / TPP;      // pairs per pass
  const int bid = blockIdx.x;
  const int ci = bid / a.batch;
  const int b = bid - ci * a.batch;
  const FFA_CONST int32_t* cp = (const FFA_CONST int32_t*)(a.combine + (int64_t)ci * kRec);
  const int q0 = cp[0], nrows = cp[1], h0 = cp[2], nch = cp[3], slot0 = cp[4];
  const int G = a.heads_per_item;
  const int npairs = nrows * G;
  const int t = threadIdx.x;
  const int dq = (t % TPP) * 4;
  // Each lane merges two (row, head) pairs per pass, p and p + PPP: the loads of
  // both are issued before either is consumed, so that twice as many partials are
  // in flight per lane.  Chunks come in groups of four (four independent loads).
  constexpr int NG = 4;
  struct Grp {
    float l[NG];
    f32x4_t x[NG];
  };
  auto load_grp = [&](int64_t base, int c, Grp& g) {
    const float* lsep = a.ws_lse + base;
    const float* op = a.ws_o + base * D + dq;
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      if (c + u < nch) {
        g.l[u] = lsep[(int64_t)(c + u) * kSlotsPerItem];
        g.x[u] = *reinterpret_cast<const f32x4_t*>(op + (int64_t)(c + u) * kSlotsPerItem * D);
      } else {
        g.l[u] = -INFINITY;
        g.x[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };
  // running (max, denominator, weighted sum) of one pair, rescaled when the max grows
  struct Acc {
    float m = -INFINITY, den = 0.0f;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  };
  auto merge = [&](Acc& r, const float (&l)[NG], const f32x4_t (&x)[NG]) {
    const float gm = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
    const float mn = fmaxf(r.m, gm);
    if (mn == -INFINITY) return;  // nothing visible yet
    const float sc = __expf(r.m - mn);  // 0 while r.m is -inf (den and acc are still 0)
    r.den *= sc;
    r.acc *= sc;
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const float w = __expf(l[u] - mn);  // 0 for an empty chunk (lse -inf)
      r.den += w;
      r.acc += w * x[u];
    }
    r.m = mn;
  };
  auto finish = [&](int p, Acc& r) {
    const int row = q0 + p / G, h = h0 + p % G;
    // sink logits: denominator terms without a value
    if (a.n_sink > 0) {
      const float* sp = a.sink + (int64_t)b * a.sk_sb + (int64_t)row * a.sk_st + (int64_t)h * a.sk_sh;
      const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4_t x0[NG] = {z, z, z, z};
      for (int s0 = 0; s0 < a.n_sink; s0 += NG) {
        float l[NG];
#pragma unroll
        for (int u = 0; u < NG; ++u) l[u] = s0 + u < a.n_sink ? sp[(int64_t)(s0 + u) * a.sk_ss] : -INFINITY;
        merge(r, l, x0);
      }
    }
    const float inv = r.den > 0.0f ? 1.0f / r.den : 0.0f;
    V4 w4;
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = (T)(r.acc[e] * inv);
    *reinterpret_cast<V4*>(a.out + (int64_t)b * a.o_sb + (int64_t)row * a.o_st + (int64_t)h * a.o_sh + dq) = w4;
    if (dq == 0)
      a.lse[(int64_t)b * a.l_sb + (int64_t)row * a.l_st + (int64_t)h * a.l_sh] =
          r.den > 0.0f ? r.m + __logf(r.den) : -INFINITY;
  };
  for (int p = t / TPP; p < npairs; p += 2 * PPP) {
    const bool two = p + PPP < npairs;  // the second pair exists
    const int64_t base0 = (int64_t)b * a.ws_slots + slot0 + p;
    Acc r0, r1;
    for (int c = 0; c < nch; c += NG) {
      Grp g0, g1;
      load_grp(base0, c, g0);
      if (two) load_grp(base0 + PPP, c, g1);
      merge(r0, g0.l, g0.x);
      if (two) merge(r1, g1.l, g1.x);
    }
    finish(p, r0);
    if (two) finish(p + PPP, r1);
  }
}


}  // namespace

static ffa_status hip_fail(hipError_t e, const char* what) {
  return ffa::set_error(FFA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

namespace {

// Enqueues the split combine of plan p over the partials at ws (fp32 out
// [batch][slots][D], then fp32 lse [batch][slots]).  Arguments already validated.
ffa_status launch_combine(const ffa::Plan& p, const int32_t* meta, int32_t batch, void* out, int64_t o_sb,
                          int64_t o_st, int64_t o_sh, float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                          const ffa_attn_extras& ex, const float* ws, hipStream_t s) {
  if (p.num_combine == 0) return FFA_OK;
  CombineArgs ca;
  ca.combine = meta + ffa::kHdr + (size_t)p.num_items * kItemRec + (size_t)p.num_runs * kRec;
  ca.ws_o = ws;
  ca.ws_lse = ws + (size_t)batch * p.num_slots * p.head_dim;
  ca.ws_slots = p.num_slots;
  ca.out = static_cast<__bf16*>(out);
  ca.lse = lse;
  ca.o_sb = o_sb; ca.o_st = o_st; ca.o_sh = o_sh;
  ca.l_sb = l_sb; ca.l_st = l_st; ca.l_sh = l_sh;
  ca.batch = batch;
  ca.heads_per_item = p.heads_per_item;
  ca.sink = ex.n_sink > 0 ? ex.sink : nullptr;
  ca.sk_sb = ex.sink_sb; ca.sk_st = ex.sink_st; ca.sk_ss = ex.sink_ss; ca.sk_sh = ex.sink_sh;
  ca.n_sink = ex.n_sink;
  const dim3 cgrid((unsigned)((int64_t)p.num_combine * batch));
  dispatch_head_dim(p.head_dim, [&](auto d_tag) {
    dispatch_dtype(ex.dtype, [&](auto t_tag) {
      hipLaunchKernelGGL((ffa_combine<decltype(d_tag)::value, decltype(t_tag)>), cgrid, dim3(256), 0, s, ca);
    });
  });
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch ffa_combine");
  return FFA_OK;
}

// Checks shared by ffa_fwd and ffa_combine: the output tensors and the workspace.
ffa_status check_outputs(const ffa::Plan& p, int32_t batch, const void* d_meta, const void* out, int64_t o_sb,
                         int64_t o_st, int64_t o_sh, const float* lse, const void* d_workspace,
                         size_t workspace_bytes) {
  if (batch < 1) return ffa::set_error(FFA_ERR_ARG, "batch must be >= 1");
  if (!d_meta) return ffa::set_error(FFA_ERR_NULL, "d_meta is NULL");
  if (p.total_q > 0 && (!out || !lse)) return ffa::set_error(FFA_ERR_NULL, "out and lse must be non-NULL");
  const int64_t ws_need = (int64_t)batch * p.workspace_bytes();
  if (ws_need > 0 && (!d_workspace || (int64_t)workspace_bytes < ws_need))
    return ffa::set_error(FFA_ERR_WORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                                 " bytes, plan needs " + std::to_string(ws_need));
  if (((uintptr_t)out & 15u) != 0) return ffa::set_error(FFA_ERR_ALIGN, "out must be 16-byte aligned");
  if ((o_sb & 7) || (o_st & 7) || (o_sh & 7))
    return ffa::set_error(FFA_ERR_ALIGN, "out strides must be multiples of 8 elements");
  return FFA_OK;
}

}  // namespace

extern "C" {

int32_t ffa_abi_version(void) { return FFA_ABI_VERSION; }

const char* ffa_status_string(ffa_status s) {
  switch (s) {
    case FFA_OK: return "ok";
    case FFA_ERR_NULL: return "null pointer";
    case FFA_ERR_SHAPE: return "unsupported shape";
    case FFA_ERR_GQA: return "heads_q not a multiple of heads_kv";
    case FFA_ERR_RANGE: return "range out of bounds";
    case FFA_ERR_MASK_TYPE: return "unsupported mask type";
    case FFA_ERR_OVERLAP: return "overlapping slices";
    case FFA_ERR_WORKSPACE: return "buffer missing or too small";
    case FFA_ERR_HIP: return "HIP runtime error";
    case FFA_ERR_HOST_OOM: return "host out of memory";
    case FFA_ERR_ALIGN: return "misaligned tensor or stride";
    case FFA_ERR_ARG: return "invalid argument";
  }
  return "unknown status";
}

const char* ffa_last_error(void) { return ffa::last_error(); }

ffa_status ffa_plan(const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* mask_types,
                    int32_t num_slices, int32_t total_q, int32_t total_k, int32_t heads_q, int32_t heads_kv,
                    int32_t head_dim, const ffa_plan_opts* opts, ffa_plan_t* plan_out) {
  ffa::clear_error();
  if (!plan_out) return ffa::set_error(FFA_ERR_NULL, "plan_out is NULL");
  *plan_out = nullptr;
  ffa_plan_opts o = {};
  if (opts) o = *opts;
  int32_t cus = o.num_cus;
  if (cus < 0) return ffa::set_error(FFA_ERR_ARG, "num_cus must be >= 0 (0: query the device)");
  if (cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  }
  ffa_plan_s* p = new (std::nothrow) ffa_plan_s;
  if (!p) return ffa::set_error(FFA_ERR_HOST_OOM, "host allocation of the plan failed");
  ffa_status st;
  try {
    st = ffa::build_plan(q_ranges, k_ranges, mask_types, num_slices, total_q, total_k, heads_q, heads_kv, head_dim,
                         o.split_tiles, o.max_splits, cus, o.flags, &p->plan);
  } catch (const std::bad_alloc&) {
    st = ffa::set_error(FFA_ERR_HOST_OOM, "host allocation failed while planning");
  }
  if (st != FFA_OK) {
    delete p;
    return st;
  }
  *plan_out = p;
  return FFA_OK;
}

ffa_status ffa_plan_info_get(ffa_plan_t plan, ffa_plan_info* info) {
  ffa::clear_error();
  if (!plan || !info) return ffa::set_error(FFA_ERR_NULL, "plan or info is NULL");
  const ffa::Plan& p = plan->plan;
  info->meta_bytes = p.meta_bytes();
  info->workspace_bytes = p.workspace_bytes();
  info->visible_pairs = p.visible_pairs;
  info->computed_pairs = p.computed_pairs;
  info->num_items = p.num_items;
  info->num_runs = p.num_runs;
  info->num_combine = p.num_combine;
  info->num_split_items = p.num_split_items;
  info->heads_per_item = p.heads_per_item;
  info->rows_per_item = p.rows_per_item;
  info->block_n = kBlockN;
  info->max_item_tiles = p.max_item_tiles;
  info->total_tiles = p.total_tiles;
  info->bwd_workspace_bytes = p.bwd_workspace_bytes();
  info->dq_tiles = p.dq_tiles;
  info->kv_tiles = p.kv_tiles;
  info->num_dq_items = p.num_dq_items;
  info->num_kv_items = p.num_kv_items;
  return FFA_OK;
}

ffa_status ffa_plan_sizes(ffa_plan_t plan, size_t* meta_bytes, size_t* workspace_bytes) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  if (meta_bytes) *meta_bytes = (size_t)plan->plan.meta_bytes();
  if (workspace_bytes) *workspace_bytes = (size_t)plan->plan.workspace_bytes();
  return FFA_OK;
}

ffa_status ffa_plan_upload(ffa_plan_t plan, void* d_meta, size_t meta_bytes, void* stream) {
  ffa::clear_error();
  if (!plan || !d_meta) return ffa::set_error(FFA_ERR_NULL, "plan or d_meta is NULL");
  const size_t need = (size_t)plan->plan.meta_bytes();
  if (meta_bytes < need)
    return ffa::set_error(FFA_ERR_WORKSPACE, "meta buffer of " + std::to_string(meta_bytes) + " bytes, plan needs " +
                                                 std::to_string(need));
  hipError_t e = hipMemcpyAsync(d_meta, plan->plan.meta.data(), need, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(meta)");
  return FFA_OK;
}

ffa_status ffa_plan_export(ffa_plan_t plan, void* h_meta, size_t meta_bytes) {
  ffa::clear_error();
  if (!plan || !h_meta) return ffa::set_error(FFA_ERR_NULL, "plan or h_meta is NULL");
  const size_t need = (size_t)plan->plan.meta_bytes();
  if (meta_bytes < need) return ffa::set_error(FFA_ERR_WORKSPACE, "host buffer too small for the plan metadata");
  std::memcpy(h_meta, plan->plan.meta.data(), need);
  return FFA_OK;
}

void ffa_plan_destroy(ffa_plan_t plan) { delete plan; }

ffa_status ffa_fwd(ffa_plan_t plan, const void* d_meta, int32_t batch, const void* q, int64_t q_sb, int64_t q_st,
                   int64_t q_sh, const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh, const void* v, int64_t v_sb,
                   int64_t v_st, int64_t v_sh, void* out, int64_t o_sb, int64_t o_st, int64_t o_sh, float* lse,
                   int64_t l_sb, int64_t l_st, int64_t l_sh, float softmax_scale, const ffa_attn_extras* extras,
                   void* d_workspace, size_t workspace_bytes, void* stream) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  const ffa::Plan& p = plan->plan;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
    return ffa::set_error(FFA_ERR_ARG, "softmax_scale must be finite and > 0");
  const ffa_status xs = ffa::check_extras(extras, p.total_q > 0);
  if (xs != FFA_OK) return xs;
  ffa_attn_extras ex = {};
  if (extras) ex = *extras;
  const ffa_status os = check_outputs(p, batch, d_meta, out, o_sb, o_st, o_sh, lse, d_workspace, workspace_bytes);
  if (os != FFA_OK) return os;
  if (p.total_q > 0 && !q) return ffa::set_error(FFA_ERR_NULL, "q must be non-NULL");
  const bool need_kv = p.total_tiles > 0;
  if (need_kv && (!k || !v)) return ffa::set_error(FFA_ERR_NULL, "k and v must be non-NULL");
  auto al16 = [](const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; };
  auto st8 = [](int64_t s) { return (s & 7) == 0; };
  if (!al16(q) || (need_kv && (!al16(k) || !al16(v))))
    return ffa::set_error(FFA_ERR_ALIGN, "q, k and v must be 16-byte aligned");
  if (!st8(q_sb) || !st8(q_st) || !st8(q_sh) || !st8(k_sb) || !st8(k_st) || !st8(k_sh) || !st8(v_sb) ||
      !st8(v_st) || !st8(v_sh))
    return ffa::set_error(FFA_ERR_ALIGN, "q, k and v strides must be multiples of 8 elements");
  // the kernels address one 64-key tile with unsigned 32-bit offsets from its first key
  const int64_t kv_lim = ((int64_t)1 << 31) / (2 * ffa::kBlockN);
  if (need_kv && (k_st < 0 || v_st < 0 || k_st >= kv_lim || v_st >= kv_lim))
    return ffa::set_error(FFA_ERR_ARG, "k / v token strides must be in [0, 2^24) elements");
  if (p.num_items == 0) return FFA_OK;
  if ((int64_t)p.num_items * batch > INT32_MAX || (int64_t)p.num_combine * batch > INT32_MAX)
    return ffa::set_error(FFA_ERR_ARG, "grid too large");

  const int32_t* meta = static_cast<const int32_t*>(d_meta);
  FwdArgs fa;
  fa.items = meta + ffa::kHdr;
  fa.runs = fa.items + (size_t)p.num_items * kItemRec;
  fa.q = static_cast<const __bf16*>(q);
  fa.k = static_cast<const __bf16*>(k);
  fa.v = static_cast<const __bf16*>(v);
  fa.out = static_cast<__bf16*>(out);
  fa.lse = lse;
  fa.q_sb = q_sb; fa.q_st = q_st; fa.q_sh = q_sh;
  fa.k_sb = k_sb; fa.k_st = k_st; fa.k_sh = k_sh;
  fa.v_sb = v_sb; fa.v_st = v_st; fa.v_sh = v_sh;
  fa.o_sb = o_sb; fa.o_st = o_st; fa.o_sh = o_sh;
  fa.l_sb = l_sb; fa.l_st = l_st; fa.l_sh = l_sh;
  fa.ws_o = static_cast<float*>(d_workspace);
  fa.ws_lse = fa.ws_o ? fa.ws_o + (size_t)batch * p.num_slots * p.head_dim : nullptr;
  fa.ws_slots = p.num_slots;
  fa.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  fa.total_k = p.total_k;
  fa.batch = batch;
  fa.heads_per_item = p.heads_per_item;
  fa.kv_ratio = p.heads_q / p.heads_kv;
  const bool cap = ex.softcap > 0.0f;
  fa.cap_log2 = cap ? (float)((double)ex.softcap * 1.4426950408889634074) : 0.0f;
  fa.cap_arg = cap ? (float)(2.0 * 1.4426950408889634074 * (double)softmax_scale / (double)ex.softcap) : 0.0f;
  fa.sink = ex.n_sink > 0 ? ex.sink : nullptr;
  fa.sk_sb = ex.sink_sb; fa.sk_st = ex.sink_st; fa.sk_ss = ex.sink_ss; fa.sk_sh = ex.sink_sh;
  fa.n_sink = ex.n_sink;

  const bool rn = (ex.flags & FFA_EXTRAS_ROUNDED_NORM) != 0;

  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)((int64_t)p.num_items * batch));
  const dim3 blk(64 * ffa::kWaves);
  dispatch_head_dim(p.head_dim, [&](auto d_tag) {
    dispatch_dtype(ex.dtype, [&](auto t_tag) {
      constexpr int D = decltype(d_tag)::value;
      using T = decltype(t_tag);
      if (rn) {
        if (cap) hipLaunchKernelGGL((ffa_fwd_main<D, true, true, T>), grid, blk, 0, s, fa);
        else hipLaunchKernelGGL((ffa_fwd_main<D, false, true, T>), grid, blk, 0, s, fa);
      } else {
        if (cap) hipLaunchKernelGGL((ffa_fwd_main<D, true, false, T>), grid, blk, 0, s, fa);
        else hipLaunchKernelGGL((ffa_fwd_main<D, false, false, T>), grid, blk, 0, s, fa);
      }
    });
  });
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch ffa_fwd_main");
  return launch_combine(p, meta, batch, out, o_sb, o_st, o_sh, lse, l_sb, l_st, l_sh, ex, fa.ws_o, s);
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept for the rest of the process.
static ffa_status scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return ffa::set_error(FFA_ERR_ARG, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return ffa::set_error(FFA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return FFA_OK;
}

ffa_status ffa_fwd_noalloc(ffa_plan_t plan, const void* d_meta, int32_t batch, const void* q, int64_t q_sb,
                           int64_t q_st, int64_t q_sh, const void* k, int64_t k_sb, int64_t k_st, int64_t k_sh,
                           const void* v, int64_t v_sb, int64_t v_st, int64_t v_sh, void* out, int64_t o_sb,
                           int64_t o_st, int64_t o_sh, float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                           float softmax_scale, const ffa_attn_extras* extras, void* stream) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  if (batch < 1) return ffa::set_error(FFA_ERR_ARG, "batch must be >= 1");
  const int64_t need = (int64_t)batch * plan->plan.workspace_bytes();
  if (need > (int64_t)FFA_NOALLOC_SCRATCH_BYTES)
    return ffa::set_error(FFA_ERR_WORKSPACE,
                          "the plan's split-K partials need " + std::to_string(need) +
                              " bytes, beyond the library scratch of " + std::to_string(FFA_NOALLOC_SCRATCH_BYTES) +
                              " bytes (use ffa_fwd with a caller workspace, or plan with fewer splits)");
  void* ws = nullptr;
  if (need > 0) {
    const ffa_status st = scratch_address(&ws);
    if (st != FFA_OK) return st;
  }
  return ffa_fwd(plan, d_meta, batch, q, q_sb, q_st, q_sh, k, k_sb, k_st, k_sh, v, v_sb, v_st, v_sh, out, o_sb, o_st,
                 o_sh, lse, l_sb, l_st, l_sh, softmax_scale, extras, ws, need > 0 ? (size_t)FFA_NOALLOC_SCRATCH_BYTES : 0,
                 stream);
}

ffa_status ffa_combine(ffa_plan_t plan, const void* d_meta, int32_t batch, void* out, int64_t o_sb, int64_t o_st,
                       int64_t o_sh, float* lse, int64_t l_sb, int64_t l_st, int64_t l_sh,
                       const ffa_attn_extras* extras, const void* d_workspace, size_t workspace_bytes, void* stream) {
  ffa::clear_error();
  if (!plan) return ffa::set_error(FFA_ERR_NULL, "plan is NULL");
  const ffa::Plan& p = plan->plan;
  const ffa_status xs = ffa::check_extras(extras, p.total_q > 0);
  if (xs != FFA_OK) return xs;
  ffa_attn_extras ex = {};
  if (extras) ex = *extras;
  const ffa_status os = check_outputs(p, batch, d_meta, out, o_sb, o_st, o_sh, lse, d_workspace, workspace_bytes);
  if (os != FFA_OK) return os;
  if ((int64_t)p.num_combine * batch > INT32_MAX) return ffa::set_error(FFA_ERR_ARG, "grid too large");
  return launch_combine(p, static_cast<const int32_t*>(d_meta), batch, out, o_sb, o_st, o_sh, lse, l_sb, l_st, l_sh,
                        ex, static_cast<const float*>(d_workspace), (hipStream_t)stream);
}

}  // extern "C"
