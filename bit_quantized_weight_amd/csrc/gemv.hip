// Dequantise-fused skinny GEMV for gfx950 (qgemv, qgemv_swiglu, qgemv_dequant,
// qgemv_probe_read).
//
// What it computes (NInfer article, section 2: the decode matmul over packed
// low-bit weights with residual add and SwiGLU fused in; "what NInfer is":
// 1 to 8 decode lanes):  y[n][m] = r[n][m] + sum_k x[n][k] * W[m][k].
//
// How it maps to the CDNA4 execution model
//   * Decode is bound by weight bytes (same section). Each wave streams 16-row
//     x 128-column tiles of packed codes with one 16-byte non-temporal buffer
//     load per lane (a contiguous 1 KiB per wave) and feeds them to
//     v_mfma_f32_16x16x32_bf16 as the B operand: n = weight row, k = 32
//     columns = one scale group. The A operand holds the activations.
//   * A rows are (slot, token) = (16/S)*slot + token with S = 16, 8, 4, 2, 1
//     slots for 1, 2, <= 4, <= 8, <= 16 tokens. Consecutive groups (NVFP4:
//     16-column blocks) go to consecutive slots, so one accumulator carries
//     S units' partial sums apart and the scale step runs once per S units.
//     Lanes that must hold zeros load from an out-of-range buffer offset,
//     which returns zeros. With one slot NVFP4 runs each block of a group
//     through its own MFMA (the other block's activation lanes masked), and
//     17 to 32 tokens take two blocks of 16 that share the decoded weights.
//   * Int group epilogue: the B operand is bf16(c + q) with c = 16 (int4) or
//     32 (int5); with D = sum x(c+q) and Db = c * sum x (one MFMA against a
//     constant c operand, shared by all tiles of the wave):
//     d*S + m*sum x = (m/c)*Db + d*(D - Db).
//   * Waves of a workgroup split K; their partial sums meet in LDS and are
//     added in wave order, so results are bitwise reproducible. The sum over
//     the two slots uses a fixed lane exchange.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>
#include <mutex>
#include <numeric>
#include <vector>

#include "device.hpp"
#include "kloop.hpp"
#include "layout.hpp"
#include "mx.hpp"
#include "qgemv.h"

namespace qg {

// The fields a wave needs to issue its first weight loads come first, so the
// kernel fetches them with one scalar load of the argument block and starts
// streaming after a single round trip (the rest arrives meanwhile).
struct GemvArgs {
  const uint8_t* wq;
  const uint8_t* ws;
  uint32_t wq_bytes, ws_bytes;
  uint32_t hi_offset;
  int KS;
  int ks_per_wave;
  int out_tiles;          // 16-row output tiles (M/16 rounded up)
  int up_tile0;           // swiglu: tile index of the first "up" row tile
  // Split remainder (frag > 1): workgroups [0, n_full) own whole row blocks;
  // workgroup n_full + b * frag + f owns K fragment f of row block n_full + b
  // (frag a power of two, 2^frag_log2). A fragment's waves take frag_kpw
  // k-steps each (enough for the largest fragment). Fragments below the
  // last publish partial sums (part) and raise a flag; the last fragment
  // (the highest workgroup of its block) adds them.
  int n_full, frag, frag_log2, frag_kpw;
  int waves;              // waves per workgroup (the block holds 64 * waves lanes)
  const uint16_t* x;      // bf16 [N][K]
  const float* res;       // [N][M] or null
  float* y;               // [N][M]  (swiglu: [N][I])
  uint32_t x_bytes, st_offset;
  int M;                  // output columns (I for swiglu)
  int K, G;               // G = K / 32 groups that hold data
  int N;
  int x_nks;              // LDS activation records per wave (XM_LDS kernels)
  // RMSNorm prologue (nsrc != null): activations are bf16(gamma * nsrc), and
  // the per-token scale 1 / sqrt(mean(nsrc^2) + eps) multiplies the dot
  // products in the epilogue
  const float* nsrc;      // [N][K] fp32
  const float* gamma;     // [K] fp32
  float eps;
  uint32_t nsrc_bytes, gamma_bytes;
  uint16_t* ybf;          // bf16 copy of the output [N][M], or null
  bool ystore;            // write the fp32 output y
  float* part;            // [(blocks - n_full) * (frag - 1)][NT * 128]
  uint32_t* pflag;        // word 0: sticky error; flags from word 64, 16 words apart
};

// Device-scope accesses for data one workgroup hands to another (they bypass
// the XCD-local L2, so a workgroup on another XCD reads the stored value)
__device__ __forceinline__ void st_f32_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f32_dev(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
constexpr uint32_t kFragSpin = 1u << 20;   // polls before a wait gives up

// bf16 round to nearest even of a finite or infinite fp32 (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// 8 activations bf16(gamma * h) of token row t, columns col..col+7 (zeros
// when !data), and their sum of squares of h added to ss
__device__ __forceinline__ u32x4 norm_chunk(__amdgpu_buffer_rsrc_t hr, __amdgpu_buffer_rsrc_t gr, int K, int t,
                                            int col, bool data, float& ss) {
  const uint32_t ho = data ? (uint32_t)(t * K + col) * 4u : kOOB;
  const uint32_t go = data ? (uint32_t)col * 4u : kOOB;
  const u32x4 h0 = ld128(hr, ho), h1 = ld128(hr, ho + 16u);
  const u32x4 g0 = ld128(gr, go), g1 = ld128(gr, go + 16u);
  // whole-vector casts: a bit cast of one element of an ext vector would
  // read the vector's first element instead
  const f32x4 ha = __builtin_bit_cast(f32x4, h0), hb = __builtin_bit_cast(f32x4, h1);
  const f32x4 ga = __builtin_bit_cast(f32x4, g0), gb = __builtin_bit_cast(f32x4, g1);
  const float hv[8] = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
  const float gv[8] = {ga[0], ga[1], ga[2], ga[3], gb[0], gb[1], gb[2], gb[3]};
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ss = fmaf(hv[e], hv[e], ss);
    b[e] = bf16_bits(gv[e] * hv[e]);
  }
  return u32x4{b[0] | b[1] << 16, b[2] | b[3] << 16, b[4] | b[5] << 16, b[6] | b[7] << 16};
}

// Sum over the 64 lanes in a fixed order (xor butterfly)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

// tokens per tile in the LDS reduction area: 16 per token block with one
// slot, else 8
template <int S, int TB = 1>
__host__ __device__ constexpr int red_tokens() { return S == 1 ? 16 * TB : 8; }

// Combine a lane's accumulators into per-(token, row) totals and write them
// to LDS as red[((wave*NT + t)*TK + token)*16 + row] (TK = red_tokens<S>());
// fixed order throughout.
template <int S, int NT, int TB = 1>
__device__ __forceinline__ void reduce_to_lds(f32x4 (&acc)[NT * TB], float* red, int wave, int lane) {
  const int r = lane & 15, s = lane >> 4;
  constexpr int RB = red_tokens<S, TB>() * 16;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float* p = red + (size_t)(wave * NT + t) * RB;
    if constexpr (S == 1) {           // one slot: register i of block b = token 16 b + 4 s + i
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[(16 * b + 4 * s + i) * 16 + r] = acc[t * TB + b][i];
    } else if constexpr (S == 16) {          // every register a different slot, token 0
      float v = (acc[t][0] + acc[t][1]) + (acc[t][2] + acc[t][3]);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) p[r] = v;
    } else if constexpr (S == 8) {    // tokens 0, 1 in registers (0, 2) and (1, 3)
      float v0 = acc[t][0] + acc[t][2], v1 = acc[t][1] + acc[t][3];
      v0 += __shfl_xor(v0, 16);
      v1 += __shfl_xor(v1, 16);
      v0 += __shfl_xor(v0, 32);
      v1 += __shfl_xor(v1, 32);
      if (lane < 16) {
        p[r] = v0;
        p[16 + r] = v1;
      }
    } else if constexpr (S == 4) {    // register i = token i, slot = s
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[t][i];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 16) p[i * 16 + r] = v;
      }
    } else {                          // S = 2: token 4*(s&1) + i, slot = s >> 1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[t][i];
        v += __shfl_xor(v, 32);
        if (lane < 32) p[(4 * s + i) * 16 + r] = v;
      }
    }
  }
}

// Activations in LDS: this wave's k-steps [ks0, ks0 + nks) as nks records
// of xs = 256 N + 16 bytes (token t's 128 bf16 at 256 t, then 16 zero bytes
// that A lanes outside the unit's slot read). Columns at or past K and
// k-steps at or past ks1 hold zeros, so the k-loop needs no masking.
__device__ __forceinline__ void stage_x(uint8_t* xl, __amdgpu_buffer_rsrc_t xr, int N, int K, int ks0, int ks1,
                                        int nks, int lane) {
  const int per = N * 16 + 1;   // 16-byte chunks per record
  const int xs = per * 16;
  const int total = nks * per;
  constexpr int B = 8;          // loads in flight per lane
  for (int i0 = 0; i0 < total; i0 += 64 * B) {
    u32x4 v[B];
    int dst[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int i = i0 + 64 * u + lane;
      const int kk = i / per, c = i - kk * per;
      const int t = c >> 4, col = (ks0 + kk) * 128 + (c & 15) * 8;
      const bool data = i < total && c < N * 16 && ks0 + kk < ks1 && col < K;
      v[u] = ld128(xr, data ? (uint32_t)(t * K + col) * 2u : kOOB);
      dst[u] = i < total ? kk * xs + c * 16 : -1;
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (dst[u] >= 0) *reinterpret_cast<u32x4*>(xl + dst[u]) = v[u];
  }
}

// stage_x for the RMSNorm prologue: token t's records come from
// bf16(gamma * nsrc[t]); the wave's sum of squares of nsrc over its k-range,
// per token, lands in ssw[t] (t < N; fixed summation order).
__device__ __forceinline__ void stage_x_norm(uint8_t* xl, __amdgpu_buffer_rsrc_t hr, __amdgpu_buffer_rsrc_t gr, int N,
                                             int K, int ks0, int ks1, int nks, int lane, float* ssw) {
  const int xs = (N * 16 + 1) * 16;       // record stride (as stage_x)
  const int per_tok = nks * 16;           // 16-byte chunks of one token over the wave's records
  for (int t = 0; t < N; ++t) {
    float ss = 0.0f;
    for (int i0 = 0; i0 < per_tok; i0 += 64 * 4) {
      u32x4 v[4];
      int dst[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 64 * u + lane;
        const int kk = i >> 4, c = i & 15;
        const int col = (ks0 + kk) * 128 + c * 8;
        const bool data = i < per_tok && ks0 + kk < ks1 && col < K;
        v[u] = norm_chunk(hr, gr, K, t, col, data, ss);
        dst[u] = i < per_tok ? kk * xs + (t * 16 + c) * 16 : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (dst[u] >= 0) *reinterpret_cast<u32x4*>(xl + dst[u]) = v[u];
    }
    ss = wave_sum(ss);
    if (lane == 0) ssw[t] = ss;
  }
  // the zero block of every record
  for (int kk = lane; kk < nks; kk += 64) *reinterpret_cast<u32x4*>(xl + kk * xs + N * 256) = u32x4{0u, 0u, 0u, 0u};
}

// Activation paths (A operands of the MFMAs):
//   XM_LDS   the wave's whole k-range of x staged in LDS up front;
//   XM_RING  a ring of kRing k-step records in LDS, refilled kRing - 1
//            k-steps ahead through registers (when the whole range does not
//            fit the LDS budget, e.g. 8 tokens over K = 5120);
//   XM_LOAD  buffer loads one k-step ahead that land out of range for lanes
//            outside the unit's slot.
constexpr int XM_LOAD = 0, XM_LDS = 1, XM_RING = 2;
constexpr int kRing = 4;
// ring record stride for S slots: room for 16 / S tokens (>= N) and the zero block
template <int S>
__host__ __device__ constexpr int ring_stride() { return (16 / S) * 256 + 16; }

// NT tiles per wave: plain GEMV uses NT output tiles, SwiGLU NT/2 gate tiles
// followed by NT/2 up tiles. S: slots (16 / S tokens per slot >= N). KPS:
// k-steps per weight prefetch buffer. XM: activation path.
// NORM: the RMSNorm prologue (a separate instantiation, so kernels without
// it keep their register budget)
// TB: blocks of 16 tokens (one slot only; 17 to 32 tokens take two, which
// share every decoded weight operand)
// Waves per SIMD the register allocation must allow: the int5 two-tile
// kernels at one and two tokens sit just past 168 VGPRs (two waves per SIMD
// instead of three) without the bound, which measured 25% slower and leaves
// the split-remainder grid too large to be resident.
template <int FMT, int NT, int S, int XM, bool NORM, int TB>
constexpr int min_waves_per_simd() {
  return (FMT == INT5 && NT == 2 && S >= 8 && XM != 2 && !NORM && TB == 1) ? 3 : 1;
}

template <int FMT, int NT, int S, int KPS, bool SWIGLU, int XM, bool NORM, int TB = 1, bool PRIO = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(min_waves_per_simd<FMT, NT, S, XM, NORM, TB>())))
void k_gemv(const uint8_t* a_wq, const uint8_t* a_ws, uint32_t a_wqb, uint32_t a_wsb, uint32_t a_hi, int a_KS,
            int a_kpw, int a_ot, int a_up, int a_nf, int a_fl, int a_fk, GemvArgs a) {
  static_assert(TB == 1 || (XM == XM_LOAD && !NORM), "token blocks load their activations directly");
  extern __shared__ __attribute__((aligned(16))) float red[];  // [W][NT][8][16], then the LDS activations
  __shared__ float s_ss[8][8];                                  // RMSNorm: [wave][token] sums of squares
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int W = a.waves;
  const int r = lane & 15, s = lane >> 4;
  constexpr int TO = SWIGLU ? NT / 2 : NT;
  constexpr int T = 16 / S;
  constexpr int TK = red_tokens<S, TB>(); // tokens per tile in the reduction area
  constexpr int RB = TK * 16;             // floats per (wave, tile) there
  using C = Cyc<FMT, S>;

  // The a_* arguments (copies of GemvArgs fields) are everything the first
  // weight loads need. As leading scalar kernel arguments they are preloaded
  // into SGPRs when the wave starts (the library is built with kernel
  // argument preloading), so a wave issues its first loads without a round
  // trip to the argument block.
  const int a_fr = 1 << a_fl;
  const __amdgpu_buffer_rsrc_t wq = make_rsrc(a_wq, a_wqb);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a_ws, a_wsb);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);

  // row block and K fragment (uniform), without branches or divisions
  const int bid = blockIdx.x;
  const bool isfrag = a_fr > 1 && bid >= a_nf;
  const int fq = bid - a_nf;
  const int rblk = isfrag ? a_nf + (fq >> a_fl) : bid;
  const int frag = isfrag ? (fq & (a_fr - 1)) : -1;
  // row tiles of this wave (clamped: out-of-range tiles compute a copy of the
  // last tile and are never stored)
  int tile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int ot = rblk * TO + (SWIGLU ? (t % TO) : t);
    ot = ot < a_ot ? ot : a_ot - 1;
    tile[t] = (SWIGLU && t >= TO) ? a_up + ot : ot;
  }

  f32x4 acc[NT * TB];
#pragma unroll
  for (int t = 0; t < NT * TB; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a fragment's K range: whole cycles, fragment f of 2^frag_log2
  constexpr int CK = C::KSTEPS;
  const int nc = (a_KS + CK - 1) / CK;
  const int kb0 = isfrag ? ((frag * nc) >> a_fl) * CK : 0;
  const int kb1 = isfrag ? min(a_KS, (((frag + 1) * nc) >> a_fl) * CK) : a_KS;
  const int kpw = isfrag ? a_fk : a_kpw;
  const int ks0 = kb0 + wave * kpw;
  const int ks1 = min(kb1, ks0 + kpw);
  // the first weight loads, before the activation set-up below reads any
  // argument of the block that is not preloaded
  Step<FMT, NT, KPS> wbuf[2];
  kloop_start<FMT, NT, S, KPS>(wbuf, wq, ws, tile, a_KS, ks0, ks1, a_hi);
  constexpr bool norm = NORM;
  static_assert(!NORM || XM != XM_LOAD, "the prologue stages its activations in LDS");
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(a.nsrc, a.nsrc_bytes);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gamma, a.gamma_bytes);
  if (lane < 8) s_ss[wave][lane] = 0.0f;  // waves with an empty k-range add nothing

  // activation lane role: A row r = slot * T + token
  const int a_tok = r % T;
  if constexpr (XM == XM_LDS || XM == XM_RING) {
    // one k-step record: token t's 128 bf16 at 256 t, then 16 zero bytes at
    // 256 N; ring records take the stride of T tokens, a compile-time
    // constant, so slot addresses fold into the LDS instructions' offsets
    const int xs = XM == XM_RING ? ring_stride<S>() : a.N * 256 + 16;
    const int nrec = XM == XM_LDS ? a.x_nks : kRing;
    uint8_t* xl = reinterpret_cast<uint8_t*>(red) + (size_t)W * NT * RB * 4 + (size_t)wave * nrec * xs;
    // per (cycle position, group): this lane's data or the record's zero
    // block. Cycles of one k-step keep the four offsets in registers; longer
    // cycles (one or two tokens) select them per read (a compare with a
    // constant and a select), which keeps 8-16 registers free
    const int sigma = r / T - ((FMT == NVFP4 && S > 1) ? (s >> 1) : 0);
    const uint32_t zoff = (uint32_t)(a.N * 256);
    const uint32_t mine = a_tok < a.N ? (uint32_t)(a_tok * 256 + s * 16) : zoff;
    const int sig = a_tok < a.N ? sigma : -1;
    constexpr int OFFC = C::KSTEPS == 1 ? 1 : 0;   // table entries kept (one-k-step cycles)
    uint32_t off_tab[OFFC ? 4 : 1];
#pragma unroll
    for (int j = 0; j < (OFFC ? 4 : 0); ++j)
      off_tab[j] = sig == slot_pos<FMT, S>(0, j) ? mine + (uint32_t)(j * 64) : zoff;
    auto off_of = [&](int c, int j) -> uint32_t {
      if constexpr (OFFC) return off_tab[j];
      else return sig == slot_pos<FMT, S>(c, j) ? mine + (uint32_t)(j * 64) : zoff;
    };
    if constexpr (XM == XM_LDS) {
      auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
        const uint8_t* rec = xl + (k - ks0) * xs;
        const int ckk = pos % C::KSTEPS;
#pragma unroll
        for (int j = 0; j < 4; ++j) A[j] = *reinterpret_cast<const bf16x8*>(rec + off_of(ckk, j));
      };
      // staged after the first weight loads are issued, so the two overlap
      auto pre = [&]() {
        if constexpr (NORM) stage_x_norm(xl, hr, gr, a.N, a.K, ks0, ks1, a.x_nks, lane, s_ss[wave]);
        else stage_x(xl, xr, a.N, a.K, ks0, ks1, a.x_nks, lane);
      };
      kloop_run<FMT, NT, S, KPS, 1, 1, false, PRIO>(wbuf, wq, ws, tile, a_KS, ks0, ks1, a_hi, acts, acc, pre);
    } else {
      // Ring slot of k-step k: (k - ks0) % kRing, which equals its trip
      // position modulo kRing (trips start at ks0 + a multiple of 2 * KPS).
      // Each lane moves two 16-byte chunks of a record (N <= 8: 16 N chunks).
      // The call that fetches A for k-step k loads record k + 3 into
      // registers; two calls later that record is written to its slot (the
      // slot last read three calls before), and one call after that it is read.
      static_assert((2 * KPS) % kRing == 0, "the ring must divide the trip");
      const int nch = a.N * 16;
      // Chunks past the record (c >= 16 N) load as zeros and are written
      // onto the record's zero block, so neither side branches per lane; the
      // second chunk is skipped (uniformly) when N <= 4.
      const bool two = nch > 64;
      const uint32_t sdst0 = (uint32_t)min(lane, nch) * 16u;   // N < 4: lanes past the record hit its zero block
      const uint32_t sdst1 = (uint32_t)min(lane + 64, nch) * 16u;
      // RMSNorm: lane chunk c always belongs to token c >> 4, so each lane sums
      // the squares of its two chunks' tokens over the k-range in ssr
      float ssr[2] = {0.0f, 0.0f};
      auto ring_load = [&](u32x4 (&v)[2], int k) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !two) { v[1] = u32x4{0u, 0u, 0u, 0u}; continue; }
          const int c = lane + 64 * h;
          const int t = c >> 4, col = k * 128 + (c & 15) * 8;
          const bool data = (c < nch) & (k < ks1) & (col < a.K);
          if constexpr (NORM) v[h] = norm_chunk(hr, gr, a.K, t, col, data, ssr[h]);
          else v[h] = ld128(xr, data ? (uint32_t)(t * a.K + col) * 2u : kOOB);
        }
      };
      auto ring_store = [&](const u32x4 (&v)[2], int slot) {
        uint8_t* rec = xl + slot * ring_stride<S>();
        *reinterpret_cast<u32x4*>(rec + sdst0) = v[0];
        if (two) *reinterpret_cast<u32x4*>(rec + sdst1) = v[1];
      };
      u32x4 stg[2][2];                 // records loaded, not yet written
      auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
        ring_store(stg[pos & 1], (pos + 1) % kRing);   // record k + 1 (loaded two calls ago)
        ring_load(stg[pos & 1], k + 3);
        const uint8_t* rec = xl + (pos % kRing) * ring_stride<S>();
        const int ckk = pos % C::KSTEPS;
#pragma unroll
        for (int j = 0; j < 4; ++j) A[j] = *reinterpret_cast<const bf16x8*>(rec + off_of(ckk, j));
      };
      auto pre = [&]() {
        // zero blocks; record ks0 written now, ks0 + 1 and ks0 + 2 staged
        if (lane < kRing) *reinterpret_cast<u32x4*>(xl + lane * ring_stride<S>() + a.N * 256) = u32x4{0u, 0u, 0u, 0u};
        u32x4 v0[2];
        ring_load(v0, ks0);
        ring_load(stg[0], ks0 + 1);
        ring_load(stg[1], ks0 + 2);
        ring_store(v0, 0);
      };
      kloop_run<FMT, NT, S, KPS, 1, 1, false, PRIO>(wbuf, wq, ws, tile, a_KS, ks0, ks1, a_hi, acts, acc, pre);
      if (NORM && ks0 < ks1) {
        // tokens (lane >> 4) and 4 + (lane >> 4): sum the 16 lanes of each row
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int d = 8; d >= 1; d >>= 1) ssr[h] += __shfl_xor(ssr[h], d);
        if ((lane & 15) == 0) {
          const int t = lane >> 4;
          if (t < a.N) s_ss[wave][t] = ssr[0];
          if (4 + t < a.N) s_ss[wave][4 + t] = ssr[1];
        }
      }
    }
  } else {
    // the lane's base offset carries its slot term; tokens >= N start past the buffer
    if constexpr (TB == 1) {
      const uint32_t xbase = (a_tok < a.N ? (uint32_t)(a_tok * a.K + 8 * s) * 2u : kAbsentRow) + lane_slot_term<FMT, S>(lane);
      auto aload = [&](int g, uint32_t adj) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, ld128s(xr, xbase + adj, (uint32_t)g * 64u));
      };
      auto acts = [&](bf16x8 (&A)[4], int k, int pos) { load_acts<FMT, S>(A, k, ks1, a.G, pos % C::KSTEPS, aload); };
      kloop_run<FMT, NT, S, KPS, 1>(wbuf, wq, ws, tile, a_KS, ks0, ks1, a_hi, acts, acc);
    } else {
      // block b's A row r = token 16 b + r (one slot: no slot term)
      uint32_t xbase[TB];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const int tk = 16 * b + a_tok;
        xbase[b] = tk < a.N ? (uint32_t)(tk * a.K + 8 * s) * 2u : kAbsentRow;
      }
      auto acts = [&](bf16x8 (&A)[TB][4], int k, int pos) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          auto aload = [&](int g, uint32_t adj) -> bf16x8 {
            return __builtin_bit_cast(bf16x8, ld128s(xr, xbase[b] + adj, (uint32_t)g * 64u));
          };
          load_acts<FMT, S>(A[b], k, ks1, a.G, pos % C::KSTEPS, aload);
        }
      };
      kloop_run<FMT, NT, S, KPS, 1, TB>(wbuf, wq, ws, tile, a_KS, ks0, ks1, a_hi, acts, acc);
    }
  }

  reduce_to_lds<S, NT, TB>(acc, red, wave, lane);
  __syncthreads();

  const int nslot = a_fr - 1;
  const size_t slot0 = frag >= 0 ? (size_t)(rblk - a_nf) * nslot : 0;
  constexpr int PS = NT * RB + (NORM ? 8 : 0);   // floats per partial slot: sums, then the RMSNorm sums of squares
  static_assert(S == 1 || PS <= 2 * 128 + 8, "partial slot larger than the workspace's (the split needs N <= 8)");
  if (frag >= 0 && frag < nslot) {
    // publish this fragment's partial sums (waves added in order) and raise its flag
    float* dst = a.part + (slot0 + frag) * PS;
    for (int o = threadIdx.x; o < NT * RB; o += blockDim.x) {
      float v = 0.f;
      for (int w = 0; w < W; ++w) v += red[(size_t)w * NT * RB + o];
      st_f32_dev(dst + o, v);
    }
    if (NORM && (int)threadIdx.x < a.N) {         // this fragment's share of each token's sum of squares
      float ss = 0.f;
      for (int w = 0; w < W; ++w) ss += s_ss[w][threadIdx.x];
      st_f32_dev(dst + NT * RB + threadIdx.x, ss);
    }
    // Publication (the ordering argument, in full, with the flag poll
    // below): the partial sums are agent-scope atomic stores, which bypass
    // the XCD-local L2 and complete at the device's coherence point; every
    // thread waits for its own to complete (s_waitcnt vmcnt(0) acknowledges
    // them), the barrier puts all of that before thread 0's flag store, so
    // the flag cannot become visible before the data. Release/acquire at
    // agent scope would add an L2 writeback and invalidate per fragment:
    // measured 2x slower for the whole launch.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(a.pflag + 64 + (slot0 + frag) * 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (frag >= 0) {
    // last fragment: wait for the others (dispatched before it), bounded
    if (wave == 0 && lane < nslot) {
      uint32_t* fl = a.pflag + 64 + (slot0 + lane) * 16;
      uint32_t it = 0;
      // The partial sums are read below with agent-scope atomic loads, which
      // go to the coherence point; they are issued only after this loop has
      // seen the flag (the branch depends on the loaded value, and the
      // signal fence keeps the compiler from moving the reads above it).
      while (__hip_atomic_load(fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (++it >= kFragSpin) {
          atomicOr(a.pflag, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __hip_atomic_store(fl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // its only reader
    }
    __syncthreads();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }

  float st = 1.0f;
  if constexpr (FMT == NVFP4) st = __builtin_bit_cast(float, ld32(ws, a.st_offset));
  // sum of a (tile, token, row) over the earlier fragments, in fragment order
  auto frag_sum = [&](int o) -> float {
    float v = 0.f;
    for (int f = 0; f < nslot; ++f) v += ld_f32_dev(a.part + (slot0 + f) * PS + o);
    return v;
  };
  const int n_out = TO * RB;
  for (int o = threadIdx.x; o < n_out; o += blockDim.x) {
    const int to = o / RB, rem = o - to * RB;
    const int tok = rem >> 4, row = rem & 15;
    const int ot = rblk * TO + to;
    const int col = ot * 16 + row;
    if (tok >= a.N || ot >= a_ot || col >= a.M) continue;
    float sc = st;                        // NVFP4 tensor scale, times the RMSNorm scale
    if constexpr (NORM) {
      float ss = 0.f;
      if (frag >= 0) ss = frag_sum(NT * RB + tok);   // the other fragments' K ranges, in fragment order
      for (int w = 0; w < W; ++w) ss += s_ss[w][tok];
      sc = sc * (1.0f / sqrtf(ss / (float)a.K + a.eps));
    }
    float v = 0.f, vo = 0.f;
    for (int w = 0; w < W; ++w) vo += red[((size_t)(w * NT + to) * TK + tok) * 16 + row];
    if (frag >= 0) {
      v = frag_sum(to * RB + rem);
      v += vo;
    } else {
      v = vo;
    }
    v *= sc;
    const size_t at = (size_t)tok * a.M + col;
    if constexpr (SWIGLU) {
      float u = 0.f, uo = 0.f;
      for (int w = 0; w < W; ++w) uo += red[((size_t)(w * NT + TO + to) * TK + tok) * 16 + row];
      if (frag >= 0) {
        u = frag_sum((TO + to) * RB + rem);
        u += uo;
      } else {
        u = uo;
      }
      u *= sc;
      v = v / (1.0f + expf(-v)) * u;
    } else {
      if (a.res) v += a.res[at];
    }
    if (a.ystore) a.y[at] = v;
    if (a.ybf) a.ybf[at] = (uint16_t)bf16_bits(v);
  }
}

// ---- debug dump: packed -> fp32 weights, bit-exact definition ---------------
// One thread per (tile, lane): 4 groups x 8 slots.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* wqp, const uint8_t* wsp, uint32_t wq_bytes,
                                                 uint32_t ws_bytes, uint32_t hi_offset, uint32_t st_offset,
                                                 int M, int K, int KS, int RT, float* out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)RT * KS * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t tau = gid >> 6;
  const int rt = (int)(tau / KS), ks = (int)(tau % KS);
  const int r = lane & 15, s = lane >> 4;
  const int row = rt * 16 + r;
  if (row >= M) return;
  const __amdgpu_buffer_rsrc_t wq = make_rsrc(wqp, wq_bytes);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(wsp, ws_bytes);
  const u32x4 cw = ld128(wq, (uint32_t)tau * (FMT == INT8 ? 2048u : 1024u) + (uint32_t)lane * 16u);
  u32x4 cw2 = {0u, 0u, 0u, 0u};
  if (FMT == INT8) cw2 = ld128(wq, (uint32_t)tau * 2048u + 1024u + (uint32_t)lane * 16u);
  uint32_t H = 0;
  if (FMT == INT5) H = ld32(wq, hi_offset + (uint32_t)tau * 256u + (uint32_t)lane * 4u);
  float st = 1.0f;
  if (FMT == NVFP4) st = __builtin_bit_cast(float, ld32(ws, st_offset));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
    bf16x8 B;
    if (FMT == INT4) B = dec_int4(v);
    else if (FMT == INT5) {
      bf16x8 B4[4];
      dec_int5_step(cw, H, B4);
      B = B4[j];
    }
    else if (FMT == INT8) {
      const u32x4 q = j < 2 ? cw : cw2;
      B = (j & 1) ? dec_int8(q.z, q.w) : dec_int8(q.x, q.y);
    } else B = dec_nvfp4(v);
    const int pos = 2 * (j & 1) + (j >> 1);
    float d = 0.f, mn = 0.f, sb = 0.f;
    if (FMT == INT4 || FMT == INT5) {
      const uint32_t dm = ld32(ws, (uint32_t)tau * 256u + (uint32_t)r * 16u + 4u * pos);
      d = f16_lo(dm);
      mn = f16_hi(dm);
    } else if (FMT == INT8) {
      const uint32_t dw = ld32(ws, (uint32_t)tau * 128u + (uint32_t)r * 8u + 4u * (pos >> 1));
      d = (pos & 1) ? f16_hi(dw) : f16_lo(dw);
    } else {
      const uint32_t sw = ld32(ws, (uint32_t)tau * 128u + (uint32_t)r * 8u + 4u * (uint32_t)(s >> 1));
      sb = j == 0 ? e4m3_byte<0>(sw) : j == 1 ? e4m3_byte<1>(sw) : j == 2 ? e4m3_byte<2>(sw) : e4m3_byte<3>(sw);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = ks * 128 + 32 * j + 8 * s + e;
      if (k >= K) continue;
      const float b = (float)B[e];
      float w;
      if (FMT == INT4) w = fmaf(d, b - 16.0f, mn);                  // d*q exact: one rounding
      else if (FMT == INT5) w = fmaf(d, b - 32.0f, mn);
      else if (FMT == INT8) w = d * b;
      else w = st * (b * sb);                                        // b*sb exact
      out[(int64_t)row * K + k] = w;
    }
  }
}

// ---- bandwidth probe -------------------------------------------------------
__global__ __launch_bounds__(256) void k_probe(const uint8_t* p, uint32_t bytes, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p, bytes);
  const uint32_t n16 = bytes / 16u;
  const uint32_t stride = gridDim.x * blockDim.x;
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3u * stride < n16; i += 4u * stride) {
    const u32x4 v0 = ld128_nt(r, i * 16u);
    const u32x4 v1 = ld128_nt(r, (i + stride) * 16u);
    const u32x4 v2 = ld128_nt(r, (i + 2u * stride) * 16u);
    const u32x4 v3 = ld128_nt(r, (i + 3u * stride) * 16u);
    acc ^= v0 ^ v1 ^ v2 ^ v3;
  }
  for (; i < n16; i += stride) acc ^= ld128_nt(r, i * 16u);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[0] = acc.x;
}

}  // namespace qg

// ============================================================================
// Host side: validation and dispatch
// ============================================================================
using namespace qg;

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int map_hip(hipError_t e) { return e == hipSuccess ? QGEMV_OK : QGEMV_EHIP; }

struct LaunchShape {
  int nt;       // tiles per wave (including up tiles for SwiGLU)
  int waves;    // waves per workgroup (<= kMaxWaves)
  int slots;    // S
  int kpw;      // k-steps per wave (a multiple of the cycle)
  int kps;      // k-steps per weight prefetch buffer
  int prio = 0; // k-loop wave priority from progress
  bool inv = false;  // batch-invariant mode (no choice that could order a sum may follow N)
};

int slots_for(int N) { return N == 1 ? 16 : N == 2 ? 8 : N <= 4 ? 4 : N <= 8 ? 2 : 1; }   // N <= 32

// k-steps per cycle for (format, slots): wave ranges are multiples of it
int cycle_ksteps(int fmt, int S) {
  const int groups = fmt == NVFP4 ? S / 2 : S;
  return groups >= 4 ? groups / 4 : 1;
}

// Launch shape: S slots from N, NT row tiles per workgroup and K split over
// its W waves. The choices come from sweeps on MI355X (the dense layer's
// three shapes and [17408][5120], every format, N = 1, 2, 4, 8):
//   * The plain GEMV takes one row tile per workgroup once the matrix has
//     enough tiles: the chip's 256 compute units then see twice as many
//     workgroups, so the share of units that get one workgroup more than the
//     others (and finish last) costs half as much. Measured 5-20% faster from
//     768 tiles at every N, and from 384 tiles at N >= 2; smaller matrices
//     (the down projection's 320 tiles) stay faster with two, except NVFP4
//     at N <= 2 and int8 at N = 2, which take one tile on every shape.
//     SwiGLU always keeps a gate tile and its up tile together.
//   * A wave streams best with 12-20 k-steps of its tiles: 20 at N = 1 and
//     N > 4; on one-tile workgroups of large matrices 20 at every N (NVFP4
//     16), on smaller ones 12 at N = 2 and for int5/int8 at N = 4, 16 for
//     int4/NVFP4 at N = 4, NVFP4 at N = 1 with 12. Gate/up pairs take
//     longer ranges: at N = 1 28 for int5/int8 (int4 20, NVFP4 24), at
//     N = 2-4 int4 20, int5/int8 40 (one wave per workgroup), NVFP4 24;
//     SwiGLU at N > 4 the whole K (one wave), long K at N > 4 five waves
//     per workgroup. With the RMSNorm
//     prologue (every wave converts and sums its own range of the source
//     row) longer ranges win: at N = 1 the whole K in one wave for int4 and
//     int5 (12% and 5% faster than 20 and 28 there), NVFP4 20, int8 28; at
//     N = 2 the whole K for int4 and int5 (13%), NVFP4 and int8 20; at N = 3-4
//     the whole K in every format with the activation ring (11-23% faster).
// The grid should hold at least ~900 waves so the chip's 1024 SIMDs have
// work; below that the k-range per wave shrinks (never under one scale
// cycle). Each wave's range is a whole number of cycles.
bool single_tile(int fmt, int N, bool swiglu, int64_t out_tiles) {
  if (swiglu || N > 8) return false;      // 9-16 tokens: two tiles share each activation load
  if ((fmt == NVFP4 && N <= 2) || (fmt == INT8 && N == 2)) return true;   // every shape
  return out_tiles >= 768 || (N >= 2 && out_tiles >= 384);
}

int ksteps_per_wave(int fmt, int N, bool swiglu, bool one_tile, int64_t KS, int64_t out_tiles, bool norm) {
  if (swiglu) {                          // gate/up pairs: [2 x 17408][5120] sweeps with the split remainder
    if (norm && N <= 4) {                // RMSNorm prologue: mostly one wave per pair
      if (N == 1) return fmt == NVFP4 ? 20 : fmt == INT8 ? 28 : 40;
      if (N == 2) return (fmt == NVFP4 || fmt == INT8) ? 20 : 40;
      return 40;                         // N = 3-4, with the activation ring (launch_s)
    }
    if (fmt == NVFP4) return N <= 4 ? 24 : 40;
    if (N == 1) return fmt == INT4 ? 20 : 28;
    if (N <= 4) return fmt == INT4 ? 20 : 40;   // int4: 20 measured 1.5-3% faster than 28 (two sweeps)
    return 40;
  }
  if (one_tile) {
    if (out_tiles >= 768) return fmt == NVFP4 ? 16 : 20;   // NVFP4 16 at every N (at N = 5-8 3-6% faster than 20)
    if (N == 1) return fmt == NVFP4 ? 12 : 20;
    if (N == 2) return fmt == INT8 ? 20 : 12;
    if (N <= 4) return (fmt == INT4 || fmt == NVFP4) ? 16 : 12;
    return 20;
  }
  if (N == 1) return 20;
  if (N == 2) return 12;
  if (N <= 4) return (fmt == INT8 || fmt == NVFP4) ? 12 : 20;
  return KS >= 64 ? (int)((KS + 4) / 5) : 20;   // long K at N > 4: five waves per workgroup
}

// Plain GEMVs on medium grids, from a sweep of one-tile workgroups over 1-8
// waves (K split evenly over the waves; MI355X, every format, N = 1, 2, 4,
// 8, on 7168 x 5120 and 5120 x 17408): one row tile per workgroup and the
// listed waves per workgroup; 6-30% faster than the general rule at N >= 4,
// within 2% of the best measured choice. int5 on the long-K shape at N = 1
// stages each wave's whole activation range (ring_first): 6% faster than its
// two-tile general rule, which the ring made slower.
//   384 <= tiles < 768, K <= 8192 (QKV-like):  four waves (int4 and NVFP4
//     at N = 1: five).
//   256 <= tiles < 384, K >= 8192 (down-like): by format and tokens below.
bool medium_grid(int fmt, int N, int64_t out_tiles, int64_t KS, int* waves) {
  if (N > 8) return false;
  if (out_tiles >= 384 && out_tiles < 768 && KS <= 64) {
    // int4 / NVFP4 at N = 1: five waves of 8 k-steps (int4 splits 40 as
    // 12 + 12 + 12 + 4 with four) measured 2-3% faster
    *waves = (N == 1 && (fmt == INT4 || fmt == NVFP4)) ? 5 : 4;
    return true;
  }
  if (out_tiles >= 256 && out_tiles < 384 && KS >= 64) {
    static const int8_t w[4][4] = {
        // N = 1, 2, 3-4, 5-8
        {7, 6, 5, 4},   // int4
        {5, 4, 4, 4},   // int5
        {5, 5, 5, 4},   // int8 (N = 1: with eight slots, pick_shape)
        {8, 6, 6, 5},   // nvfp4
    };
    const int nb = N == 1 ? 0 : N == 2 ? 1 : N <= 4 ? 2 : 3;
    *waves = w[fmt - INT4][nb];
    return *waves > 0;
  }
  return false;
}

constexpr size_t kMaxLdsActs = 48 * 1024;
constexpr size_t kMaxLdsNorm = 64 * 1024;   // RMSNorm prologue: the ring may use up to this
constexpr int kMaxWaves = 8;
constexpr int64_t kMinGridWaves = 900;

// Batch-invariant mode: every choice that orders a token's sums (the slot
// count, hence the scale-step cycles and the lane reduction, and the K split
// over waves) depends on K alone, so a token's outputs are the same bits for
// any N; the row tiles per workgroup (which do not touch the order) still
// follow N.
constexpr int kInvariantKsteps = 20;

LaunchShape pick_shape(int fmt, int64_t KS, int64_t out_tiles, int N, bool swiglu, bool norm, bool inv) {
  LaunchShape ls;
  ls.kps = 2;
  ls.slots = inv ? 2 : slots_for(N);
  // int8 on the down-like grid at N = 1: eight slots (two-k-step scale
  // cycles) and five waves measured 6% faster than sixteen slots and four
  int mw8 = 0;
  if (!inv && !swiglu && N == 1 && fmt == INT8 && out_tiles < 384 && medium_grid(fmt, N, out_tiles, KS, &mw8))
    ls.slots = 8;
  if (inv) {
    ls.inv = true;
    const bool one = single_tile(fmt, N, swiglu, out_tiles);
    ls.nt = one ? 1 : 2;
    int64_t kpw = kInvariantKsteps;   // the slot count 2 has one-k-step cycles in every format
    while ((KS + kpw - 1) / kpw > kMaxWaves) ++kpw;
    if (norm) {                       // LDS ring budget, taken at two tiles so that it does not depend on N
      const int64_t ring = 4 * (8 * 256 + 16) + 2 * 512;
      while ((KS + kpw - 1) / kpw * ring > (int64_t)kMaxLdsNorm && kpw < KS) ++kpw;
    }
    ls.waves = (int)((KS + kpw - 1) / kpw);
    ls.kpw = (int)kpw;
    return ls;
  }
  const int cyc = cycle_ksteps(fmt, ls.slots);
  auto waves_for = [&](int64_t kpw) { return (KS + kpw - 1) / kpw; };
  auto round_cyc = [&](int64_t kpw) { return (kpw + cyc - 1) / cyc * cyc; };
  int64_t kpw;
  int mw = 0;
  if (!swiglu && medium_grid(fmt, N, out_tiles, KS, &mw)) {
    ls.nt = 1;
    kpw = round_cyc((KS + mw - 1) / mw);
    // progress priority (kloop_run): on the long-K shape at N = 1 int5 (five
    // waves per workgroup) measured 4% faster, NVFP4 (eight) 3.5%; int4,
    // int8, N >= 2, the QKV-like shape and gate/up pairs gained nothing or lost
    ls.prio = N == 1 && KS >= 64 && out_tiles < 384 && (fmt == INT5 || fmt == NVFP4);
  } else {
    const bool one = single_tile(fmt, N, swiglu, out_tiles);
    ls.nt = one ? 1 : 2;
    const int per = ksteps_per_wave(fmt, N, swiglu, one, KS, out_tiles, norm);
    const int64_t to = swiglu ? ls.nt / 2 : ls.nt;     // output tiles per workgroup
    const int64_t wgs = (out_tiles + to - 1) / to;
    kpw = round_cyc(per);
    while (kpw > cyc && wgs * waves_for(kpw) < kMinGridWaves) kpw = round_cyc(kpw - cyc > cyc ? kpw - cyc : cyc);
  }
  while (waves_for(kpw) > kMaxWaves) kpw += cyc;
  if (norm) {
    // the RMSNorm prologue stages activations in LDS: keep the ring within budget
    const int64_t ring = 4 * ((16 / ls.slots) * 256 + 16) + ls.nt * 512;
    while (waves_for(kpw) * ring > (int64_t)kMaxLdsNorm && kpw < KS) kpw += cyc;
  }
  ls.waves = (int)waves_for(kpw);
  ls.kpw = (int)kpw;
  return ls;
}

// At N <= 4 a wave's activations could be staged whole in LDS before its
// k-loop or stream through the four-record ring; the ring measured 2-20%
// faster on the dense layer's shapes (every format, N = 1, 2, 4), except
// for the int5 and int8 gate/up pairs and the int formats' two-tile long-K
// projection (the down projection) at N = 1, and int5's one-tile long-K
// projection at N = 1, which keep the whole range.
bool ring_first(int fmt, int N, bool swiglu, int nt, int64_t KS) {
  if (N == 1 && swiglu && (fmt == INT5 || fmt == INT8)) return false;
  if (N == 1 && !swiglu && KS >= 64 && (nt == 2 ? fmt != NVFP4 : fmt == INT5)) return false;
  return true;
}


// Split remainder. With B row blocks on C compute units, B mod C blocks
// would leave that many units with one workgroup more than the rest, and
// the launch ends when those finish. The first floor(B / C) C blocks stay
// whole; each remaining block's K range is cut into F = C / gcd(B mod C, C)
// fragments, so every unit receives the same weight bytes. Taken when
// B mod C <= C / 2 (a larger remainder already keeps most units busy to
// the end, and the fragments' own cost won: measured on [7168][5120]),
// F <= kMaxFrag, a fragment still gives each wave at least one scale cycle,
// and every workgroup of the split grid is resident at once. The last fragment of a block adds the others' partial sums in
// fragment order, so results are reproducible, but their bits differ from
// the unsplit sum.
constexpr int kMaxFrag = 8;
constexpr int64_t kSplitHeader = 256;     // sticky error word, then padding

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) return 0;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// flag words (64 bytes each) and partial-sum slots (NT <= 2 tiles of 8 x 16
// floats, then 8 RMSNorm sums of squares)
constexpr int64_t kSlotFloats = 2 * 128 + 8;
int64_t split_slots(int cus) { return (int64_t)(kMaxFrag - 1) * cus; }
int64_t split_flag_bytes(int cus) { return (kSplitHeader + 64 * split_slots(cus) + 255) / 256 * 256; }
int64_t split_bytes(int cus) { return split_flag_bytes(cus) + split_slots(cus) * kSlotFloats * 4; }

void plan_split(int fmt, const LaunchShape& ls, bool swiglu, int64_t out_tiles, int64_t KS, int cus, GemvArgs& a) {
  a.n_full = 0;
  a.frag = 1;
  a.frag_log2 = 0;
  a.frag_kpw = 0;
  if (cus < 1) return;
  const int64_t to = swiglu ? ls.nt / 2 : ls.nt;
  const int64_t blocks = (out_tiles + to - 1) / to;
  const int64_t n_full = blocks / cus * cus, r = blocks - n_full;
  if (r == 0 || 2 * r > cus) return;
  const int64_t F = cus / std::gcd(r, (int64_t)cus);
  if (F > kMaxFrag || (F & (F - 1))) return;        // the kernel divides by shifts
  const int cyc = cycle_ksteps(fmt, ls.slots);
  const int64_t nc = (KS + cyc - 1) / cyc;
  if (nc / F < ls.waves) return;
  int lg = 0;
  while ((int64_t(1) << lg) < F) ++lg;
  // k-steps per wave that cover the largest fragment (never more than the
  // unsplit range, which sizes the LDS activation records)
  int64_t kpw = 0;
  for (int64_t f = 0; f < F; ++f) {
    const int64_t b0 = ((f * nc) >> lg) * cyc, b1 = std::min(KS, (((f + 1) * nc) >> lg) * cyc);
    const int64_t c = ((b1 - b0 + cyc - 1) / cyc + ls.waves - 1) / ls.waves * cyc;
    kpw = std::max(kpw, c);
  }
  if (kpw > ls.kpw) return;
  a.n_full = (int)n_full;
  a.frag = (int)F;
  a.frag_log2 = lg;
  a.frag_kpw = (int)kpw;
}

using KernelFn = void (*)(const uint8_t*, const uint8_t*, uint32_t, uint32_t, uint32_t, int, int, int, int, int, int,
                          int, GemvArgs);

// Workgroups of a kernel resident per compute unit (cached per device, kernel,
// block size and LDS bytes); 0 if the runtime cannot say.
int resident_per_cu(const void* fn, int threads, size_t lds) {
  struct Entry { const void* fn; int threads; size_t lds; int dev; int n; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.fn == fn && e.threads == threads && e.lds == lds && e.dev == dev) return e.n;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess) n = 0;
  cache.push_back(Entry{fn, threads, lds, dev, n});
  return n;
}

template <int FMT, int NT, int S, int KPS>
hipError_t launch_s(const GemvArgs& a0, const LaunchShape& ls, bool swiglu, hipStream_t stream) {
  const int TO = swiglu ? NT / 2 : NT;
  const int64_t blocks = (a0.out_tiles + TO - 1) / TO;
  const dim3 block((unsigned)(64 * ls.waves));
  GemvArgs a = a0;
  a.waves = ls.waves;
  const int U = 2 * KPS;   // k-steps per trip of the k-loop
  a.x_nks = (ls.kpw + U - 1) / U * U + 1;
  const size_t rec = (size_t)a.N * 256 + 16;
  const bool two_blocks = S == 1 && a.N > 16;   // 17 to 32 tokens: two blocks of 16
  const size_t red = (size_t)ls.waves * NT * red_tokens<S>() * (two_blocks ? 2 : 1) * 16 * sizeof(float);
  const size_t whole = (size_t)ls.waves * a.x_nks * rec, ring = (size_t)ls.waves * kRing * ring_stride<S>();
  // (the ring moves at most 8 tokens per record: one slot's 16 load directly)
  int xm = whole <= kMaxLdsActs ? XM_LDS : ((ring <= kMaxLdsActs && S > 1) ? XM_RING : XM_LOAD);
  if (xm == XM_LDS && S >= 4 && !a.nsrc && ring <= kMaxLdsActs && ring_first(FMT, a.N, swiglu, NT, a.KS))
    xm = XM_RING;
  if (two_blocks) xm = XM_LOAD;
  // gate/up pairs at N = 5-8 (two slots) read their activations straight from
  // memory: int4 9-10% and int5 3-4% faster than the ring, NVFP4 1-4%; int8,
  // and every plain GEMV shape measured, keep the staged paths
  if (swiglu && S == 2 && a.N >= 5 && FMT != INT8 && !a.nsrc) xm = XM_LOAD;
  // the RMSNorm prologue for gate/up pairs at N = 3-4 streams through the ring
  // (not in batch-invariant mode: the two paths add a row's squares in
  // different orders)
  if (a.nsrc && swiglu && !ls.inv && a.N >= 3 && a.N <= 4 && xm == XM_LDS && S > 1 && red + ring <= kMaxLdsNorm)
    xm = XM_RING;
  if (a.nsrc && xm == XM_LOAD) {         // the RMSNorm prologue stages its activations in LDS
    if (red + ring > kMaxLdsNorm) return hipErrorNotSupported;
    xm = XM_RING;
  }
  const size_t lds = red + (xm == XM_LDS ? whole : (xm == XM_RING ? ring : 0));
  const bool norm = a.nsrc != nullptr;
  KernelFn fn = nullptr;
#define QG_PICK(SW, XMV, NRM) fn = k_gemv<FMT, NT, S, KPS, SW, XMV, NRM>
  if (NT >= 2 && swiglu) {
    if constexpr (NT >= 2) {
      if (xm == XM_LDS) {
        if constexpr (S > 1) { if (norm) QG_PICK(true, XM_LDS, true); else QG_PICK(true, XM_LDS, false); }
        else QG_PICK(true, XM_LDS, false);
      }
      else if (xm == XM_RING) {
        if constexpr (S > 1) { if (norm) QG_PICK(true, XM_RING, true); else QG_PICK(true, XM_RING, false); }
      }
      else QG_PICK(true, XM_LOAD, false);
    }
  } else {
    if (xm == XM_LDS) {
      if constexpr (S > 1) { if (norm) QG_PICK(false, XM_LDS, true); else QG_PICK(false, XM_LDS, false); }
      else QG_PICK(false, XM_LDS, false);
    }
    else if (xm == XM_RING) {
      if constexpr (S > 1) { if (norm) QG_PICK(false, XM_RING, true); else QG_PICK(false, XM_RING, false); }
    }
    else QG_PICK(false, XM_LOAD, false);
  }
#undef QG_PICK
  if constexpr (S == 1 && NT >= 2) {
    // SwiGLU with 17 to 32 tokens: two token blocks share each decoded weight
    // operand (the plain GEMV runs two launches instead)
    if (two_blocks) fn = swiglu ? (KernelFn)k_gemv<FMT, NT, 1, KPS, true, XM_LOAD, false, 2> : nullptr;
  }
  if constexpr (NT == 1 && S == 16 && (FMT == INT5 || FMT == NVFP4)) {
    // the k-loop with progress priority (pick_shape decides where)
    if (ls.prio && !swiglu && !norm && (xm == XM_LDS || xm == XM_RING))
      fn = xm == XM_LDS ? (KernelFn)k_gemv<FMT, 1, 16, KPS, false, XM_LDS, false, 1, true>
                        : (KernelFn)k_gemv<FMT, 1, 16, KPS, false, XM_RING, false, 1, true>;
  }
  if (!fn) return hipErrorNotSupported;
  int64_t nwg = blocks;
  if (a.frag > 1) {
    // split only when every workgroup of the split grid is resident at once:
    // in a second dispatch round the waiting workgroups hold the units idle
    const int64_t g = a.n_full + (blocks - a.n_full) * a.frag;
    if (g <= (int64_t)resident_per_cu(reinterpret_cast<const void*>(fn), (int)block.x, lds) * device_cus()) {
      nwg = g;
    } else {
      a.frag = 1;
      a.frag_log2 = 0;
      a.n_full = 0;
    }
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)nwg), block, lds, stream, a.wq, a.ws, a.wq_bytes, a.ws_bytes, a.hi_offset, a.KS,
                     a.ks_per_wave, a.out_tiles, a.up_tile0, a.n_full, a.frag_log2, a.frag_kpw, a);
  return hipGetLastError();
}

template <int FMT, int NT, int KPS>
hipError_t launch_k(const GemvArgs& a, const LaunchShape& ls, bool swiglu, hipStream_t stream) {
  switch (ls.slots) {
    case 16: return launch_s<FMT, NT, 16, KPS>(a, ls, swiglu, stream);
    case 1: return launch_s<FMT, NT, 1, KPS>(a, ls, swiglu, stream);
    case 8: return launch_s<FMT, NT, 8, KPS>(a, ls, swiglu, stream);
    case 4: return launch_s<FMT, NT, 4, KPS>(a, ls, swiglu, stream);
    default: return launch_s<FMT, NT, 2, KPS>(a, ls, swiglu, stream);
  }
}

// Two k-steps per weight buffer. Four (twice the loads in flight per wave)
// measured 15-60% slower on one-tile workgroups and 2.7-4x slower on
// two-tile ones, although a plain streaming probe at the same waves per SIMD
// reads faster with four loads in flight than with two.
template <int FMT>
hipError_t launch_gemv(const GemvArgs& a, const LaunchShape& ls, bool swiglu, hipStream_t stream) {
  if (ls.nt == 1) return launch_k<FMT, 1, 2>(a, ls, false, stream);   // plain GEMV only
  return launch_k<FMT, 2, 2>(a, ls, swiglu, stream);
}

int validate_common(int fmt, const void* wq, const void* ws, int64_t M, int64_t K, int N, Geom* g) {
  if (fmt < INT4 || fmt > NVFP4) return QGEMV_EFORMAT;
  if (!wq || !ws) return QGEMV_EINVAL;
  if (M < 1 || K < 32 || M > (1 << 24)) return QGEMV_EINVAL;
  if (K % 32) return QGEMV_EALIGN;
  if (N < 1 || N > 32) return QGEMV_EUNSUPPORTED;
  if (!aligned16(wq) || !aligned16(ws)) return QGEMV_EALIGN;
  if (!geom(fmt, M, K, g)) return QGEMV_EINVAL;
  if (g->wq_bytes >= (1ull << 32) || g->ws_bytes >= (1ull << 32)) return QGEMV_EUNSUPPORTED;
  if ((uint64_t)N * (uint64_t)K * 2ull >= (1ull << 25)) return QGEMV_EUNSUPPORTED;  // activation bytes < 2^25
  if (g->wq_bytes >= (1ull << 31) || g->ws_bytes >= (1ull << 31)) return QGEMV_EUNSUPPORTED;
  return QGEMV_OK;
}

// fz: optional fusions (RMSNorm prologue, bf16 output), or null
int run_gemv(int fmt, const void* wq, const void* ws, const void* x, const float* res, float* y, int64_t Mout,
             int64_t Mpacked, int64_t K, int N, bool swiglu, const qgemv_fusion* fz, hipStream_t stream) {
  Geom g;
  int rc = validate_common(fmt, wq, ws, Mpacked, K, N, &g);
  if (rc) return rc;
  const bool norm = fz && fz->norm_src;
  uint16_t* ybf = fz ? fz->out_bf16 : nullptr;
  // 9 to 32 tokens use one slot: no RMSNorm prologue and no batch-invariant order
  if (N > 8 && (norm || (fz && (fz->flags & QGEMV_BATCH_INVARIANT)))) return QGEMV_EUNSUPPORTED;
  if (!swiglu && N > 16) {
    // plain GEMV: two launches of at most 16 tokens (measured faster than one
    // launch with two token blocks, whose activation loads per weight byte
    // double on one-tile workgroups)
    if (x && !aligned16(x)) return QGEMV_EALIGN;
    if ((y && !aligned4(y)) || (res && !aligned4(res)) || ((uintptr_t)ybf & 1u)) return QGEMV_EALIGN;
    qgemv_fusion f2 = fz ? *fz : qgemv_fusion{};
    int rc2 = run_gemv(fmt, wq, ws, x, res, y, Mout, Mpacked, K, 16, swiglu, fz, stream);
    if (rc2) return rc2;
    if (ybf) f2.out_bf16 = ybf + (size_t)16 * Mout;
    return run_gemv(fmt, wq, ws, x ? (const uint16_t*)x + (size_t)16 * K : nullptr, res ? res + (size_t)16 * Mout : nullptr,
                    y ? y + (size_t)16 * Mout : nullptr, Mout, Mpacked, K, N - 16, swiglu, fz ? &f2 : nullptr, stream);
  }
  if (!norm && !x) return QGEMV_EINVAL;
  if (!y && !ybf) return QGEMV_EINVAL;
  if (x && !aligned16(x)) return QGEMV_EALIGN;
  if ((y && !aligned4(y)) || (res && !aligned4(res)) || ((uintptr_t)ybf & 1u)) return QGEMV_EALIGN;
  if (norm) {
    if (!fz->norm_gamma) return QGEMV_EINVAL;
    if (!aligned16(fz->norm_src) || !aligned16(fz->norm_gamma)) return QGEMV_EALIGN;
    if (!(fz->norm_eps >= 0.0f) || fz->norm_eps > 3.0e38f) return QGEMV_EINVAL;
  }
  GemvArgs a;
  a.wq = (const uint8_t*)wq;
  a.ws = (const uint8_t*)ws;
  a.x = (const uint16_t*)x;
  a.res = res;
  a.y = y;
  a.wq_bytes = (uint32_t)g.wq_bytes;
  a.ws_bytes = (uint32_t)g.ws_bytes;
  a.x_bytes = x ? (uint32_t)((int64_t)N * K * 2) : 0u;
  a.hi_offset = (uint32_t)g.hi_offset;
  a.st_offset = (uint32_t)g.st_offset;
  a.M = (int)Mout;
  a.K = (int)K;
  a.KS = (int)g.KS;
  a.G = (int)(K / 32);
  a.N = N;
  a.out_tiles = (int)((Mout + 15) / 16);
  a.up_tile0 = swiglu ? (int)(Mout / 16) : 0;
  a.nsrc = norm ? fz->norm_src : nullptr;
  a.gamma = norm ? fz->norm_gamma : nullptr;
  a.eps = norm ? fz->norm_eps : 0.0f;
  a.nsrc_bytes = norm ? (uint32_t)((int64_t)N * K * 4) : 0u;
  a.gamma_bytes = norm ? (uint32_t)(K * 4) : 0u;
  a.ybf = ybf;
  a.ystore = y != nullptr;
  const bool inv = fz && (fz->flags & QGEMV_BATCH_INVARIANT);
  if (fz && (fz->flags & ~QGEMV_BATCH_INVARIANT)) return QGEMV_EINVAL;
  const LaunchShape ls = pick_shape(fmt, g.KS, a.out_tiles, N, swiglu, norm, inv);
  a.ks_per_wave = ls.kpw;
  a.n_full = 0;
  a.frag = 1;
  a.frag_log2 = 0;
  a.frag_kpw = 0;
  a.part = nullptr;
  a.pflag = nullptr;
  if (fz && fz->workspace) {
    const int cus = device_cus();
    if (cus < 1) return QGEMV_EHIP;
    if (!aligned16(fz->workspace) || ((uintptr_t)fz->workspace & 255u)) return QGEMV_EALIGN;
    if (fz->workspace_bytes < (size_t)split_bytes(cus)) return QGEMV_EWORKSPACE;
    if (!inv && N <= 8) plan_split(fmt, ls, swiglu, a.out_tiles, g.KS, cus, a);
    a.pflag = (uint32_t*)fz->workspace;
    a.part = (float*)((uint8_t*)fz->workspace + split_flag_bytes(cus));
  }
  hipError_t e;
  switch (fmt) {
    case INT4: e = launch_gemv<INT4>(a, ls, swiglu, stream); break;
    case INT5: e = launch_gemv<INT5>(a, ls, swiglu, stream); break;
    case INT8: e = launch_gemv<INT8>(a, ls, swiglu, stream); break;
    default: e = launch_gemv<NVFP4>(a, ls, swiglu, stream); break;
  }
  if (e == hipErrorNotSupported) return QGEMV_EUNSUPPORTED;
  return map_hip(e);
}

}  // namespace

extern "C" const char* qgemv_strerror(int status) {
  switch (status) {
    case QGEMV_OK: return "success";
    case QGEMV_EINVAL: return "invalid argument (null pointer, bad size or non-finite weights)";
    case QGEMV_EFORMAT: return "unknown weight format";
    case QGEMV_EALIGN: return "pointer or shape alignment violated";
    case QGEMV_ERANGE: return "a scale field overflows its encoding";
    case QGEMV_EWORKSPACE: return "workspace missing or too small";
    case QGEMV_EHIP: return "HIP runtime error at launch";
    case QGEMV_EUNSUPPORTED: return "size outside the supported range";
    default: return "unknown status";
  }
}

extern "C" int qgemv_version(void) { return 100; }

extern "C" int qgemv(int fmt, const void* wq, const void* ws, const void* x, const float* residual, float* y,
                     int64_t M, int64_t K, int N, hipStream_t stream) {
  if (!y) return QGEMV_EINVAL;
  return run_gemv(fmt, wq, ws, x, residual, y, M, M, K, N, false, nullptr, stream);
}

extern "C" int qgemv_swiglu(int fmt, const void* wq, const void* ws, const void* x, float* h, int64_t I, int64_t K,
                            int N, hipStream_t stream) {
  if (I < 1) return QGEMV_EINVAL;
  if (I % 16) return QGEMV_EALIGN;
  if (!h) return QGEMV_EINVAL;
  return run_gemv(fmt, wq, ws, x, nullptr, h, I, 2 * I, K, N, true, nullptr, stream);
}

extern "C" int qgemv_split_workspace_bytes(size_t* bytes) {
  if (!bytes) return QGEMV_EINVAL;
  const int cus = device_cus();
  if (cus < 1) return QGEMV_EHIP;
  *bytes = (size_t)split_bytes(cus);
  return QGEMV_OK;
}

extern "C" int qgemv_ex(int fmt, const void* wq, const void* ws, const void* x, const float* residual, float* y,
                        int64_t M, int64_t K, int N, const qgemv_fusion* fusion, hipStream_t stream) {
  return run_gemv(fmt, wq, ws, x, residual, y, M, M, K, N, false, fusion, stream);
}

extern "C" int qgemv_swiglu_ex(int fmt, const void* wq, const void* ws, const void* x, float* h, int64_t I,
                               int64_t K, int N, const qgemv_fusion* fusion, hipStream_t stream) {
  if (I < 1) return QGEMV_EINVAL;
  if (I % 16) return QGEMV_EALIGN;
  return run_gemv(fmt, wq, ws, x, nullptr, h, I, 2 * I, K, N, true, fusion, stream);
}

extern "C" int qgemv_dequant(int fmt, const void* wq, const void* ws, int64_t M, int64_t K, float* w_out,
                             hipStream_t stream) {
  if (fmt < INT4 || fmt > MXFP8) return QGEMV_EFORMAT;
  if (!wq || !ws || !w_out) return QGEMV_EINVAL;
  if (M < 1 || K < 32) return QGEMV_EINVAL;
  if (K % 32) return QGEMV_EALIGN;
  if (!aligned16(wq) || !aligned16(ws) || !aligned4(w_out)) return QGEMV_EALIGN;
  if (fmt == MXFP4 || fmt == MXFP8) return mx_dequant(fmt, wq, ws, M, K, w_out, stream);
  Geom g;
  if (!geom(fmt, M, K, &g)) return QGEMV_EINVAL;
  if (g.wq_bytes >= (1ull << 32) || g.ws_bytes >= (1ull << 32)) return QGEMV_EUNSUPPORTED;
  const int64_t threads = g.RT * g.KS * 64;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  const uint8_t* q = (const uint8_t*)wq;
  const uint8_t* s = (const uint8_t*)ws;
  const uint32_t a = (uint32_t)g.wq_bytes, b = (uint32_t)g.ws_bytes;
  const uint32_t ho = (uint32_t)g.hi_offset, so = (uint32_t)g.st_offset;
  const int Mi = (int)M, Ki = (int)K, KSi = (int)g.KS, RTi = (int)g.RT;
  switch (fmt) {
    case INT4: hipLaunchKernelGGL(k_dequant<INT4>, grid, block, 0, stream, q, s, a, b, ho, so, Mi, Ki, KSi, RTi, w_out); break;
    case INT5: hipLaunchKernelGGL(k_dequant<INT5>, grid, block, 0, stream, q, s, a, b, ho, so, Mi, Ki, KSi, RTi, w_out); break;
    case INT8: hipLaunchKernelGGL(k_dequant<INT8>, grid, block, 0, stream, q, s, a, b, ho, so, Mi, Ki, KSi, RTi, w_out); break;
    default: hipLaunchKernelGGL(k_dequant<NVFP4>, grid, block, 0, stream, q, s, a, b, ho, so, Mi, Ki, KSi, RTi, w_out); break;
  }
  return map_hip(hipGetLastError());
}

extern "C" int qgemv_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0) return QGEMV_EINVAL;
  if (bytes % 16 || !aligned16(buf) || !aligned4(sink)) return QGEMV_EALIGN;
  if (bytes >= (1ull << 32)) return QGEMV_EUNSUPPORTED;
  hipLaunchKernelGGL(k_probe, dim3(8192), dim3(256), 0, stream, (const uint8_t*)buf, (uint32_t)bytes, sink);
  return map_hip(hipGetLastError());
}
