// MX (microscaling) path on gfx950: MXFP8 / MXFP4 weights times MXFP8
// activations on the block-scaled MFMA, and the dynamic activation quantiser
// that feeds it (Decapybara page, kernel list: an MXFP8 block-scaled GEMV
// and a dynamic 32-element MXFP8 activation quantiser). Format: the public
// OCP microscaling definitions (one E8M0 scale per 32 values along K).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a 16x128 A by a 128x16 B
// whose elements are FP8 / FP4 codes, each 32-block along K scaled by an E8M0
// byte, and accumulates in fp32. Operand registers (measured on MI355X):
//   FP8 operand, lane l (row l % 16, g = l / 16): bytes 0..15 hold K 16g..16g+15,
//     bytes 16..31 hold K 64+16g..64+16g+15;
//   FP4 operand, lane l: 16 bytes hold K 32g..32g+31, low nibble first;
//   scale register of lane l: the E8M0 byte of (row l % 16, 32-block g).
// A = activations (rows = tokens, N <= 16), B = weights (16 rows per tile),
// so one MFMA per tile and k-step covers every token: there is no decode.
// The weight layout (layout.hpp) stores each lane's operand bytes
// contiguously; activation codes stay row-major [N][K], whose 16-byte runs
// are the A operand's halves as they are.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "layout.hpp"
#include "mx.hpp"
#include "qgemv.h"

namespace qg {

typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ uint32_t ld8s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// ---- MXFP8 quantisation (OCP microscaling) --------------------------------
// E4M3 code of an fp32 value: nearest, ties to even, saturating at 448, sign
// bit kept (NaN stays NaN). Every step below is exact except the one rintf.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  const uint32_t sign = (__float_as_uint(t) >> 24) & 0x80u;
  const float a = fabsf(t);
  uint32_t code;
  if (a != a) {
    code = 0x7Fu;
  } else if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                  // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);        // 8 rounds up to the least normal, code 8
  } else {
    const int e = (int)(__float_as_uint(a) >> 23) - 127;                  // floor(log2 a), -6..8
    const float f = a * __uint_as_float((uint32_t)(127 - e) << 23);       // in [1, 2)
    code = (uint32_t)(((e + 7) << 3) + (int)rintf((f - 1.0f) * 8.0f));    // carries into e + 1
    code = min(code, 0x7Eu);
  }
  return sign | code;
}

// Eight lanes per MX block of 32 bf16 values, four values each: the block's
// amax comes from the bf16 magnitudes as integers (their order is the
// values') combined over the eight lanes, X = floor(log2 amax) - 8 clamped
// to [-127, 127] (a bf16 subnormal amax has floor(log2) < -126, so it
// clamps too), and each lane converts its four values scaled by 2^-X
// (exact) into four E4M3 bytes.
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t* x, int64_t nblk, uint8_t* codes, uint8_t* scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = t >> 3;                 // block; its 8 lanes share i, so they leave together
  if (i >= nblk) return;
  const u32x2 v = *reinterpret_cast<const u32x2*>(x + t * 4);
  uint32_t m = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 8));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 8));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4, 8));
  int X = (int)(m >> 7) - 127 - 8;
  X = m == 0 ? -127 : max(-127, min(127, X));
  const float sc = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X (X <= 120 for bf16 inputs)
  const uint32_t c = e4m3_rne_sat(__uint_as_float(v.x << 16) * sc) | (e4m3_rne_sat(__uint_as_float(v.x & 0xFFFF0000u) * sc) << 8) |
                     (e4m3_rne_sat(__uint_as_float(v.y << 16) * sc) << 16) |
                     (e4m3_rne_sat(__uint_as_float(v.y & 0xFFFF0000u) * sc) << 24);
  *reinterpret_cast<uint32_t*>(codes + t * 4) = c;
  if ((t & 7) == 0) scales[i] = (uint8_t)(X + 127);
}

// ---- the block-scaled GEMV -------------------------------------------------
struct MxArgs {
  const uint8_t* wq;
  const uint8_t* ws;
  const uint8_t* xq;      // [N][K] E4M3 codes
  const uint8_t* xs;      // [N][K/32] E8M0
  const float* res;       // [N][M] or null (may alias y)
  float* y;               // [N][M]
  uint32_t wq_bytes, ws_bytes, xq_bytes, xs_bytes;
  int M, K, KS, G, N, out_tiles, ks_per_wave;
  int up_tile0;           // SwiGLU: row tile of the first up row (gate rows come first)
  uint8_t* hq;            // SwiGLU with quantised output: [N][M] E4M3 codes of bf16(h)
  uint8_t* hs;            // and their E8M0 scales [N][M/32] (y, if not null, receives h too)
};

// bf16 bits of an fp32 value, round to nearest even
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// operands of one k-step: activations of TB blocks of 16 tokens (shared by
// the tiles) and NT weight tiles
template <int FMT, int NT, int TB>
struct MxStep {
  u32x4 a0[TB], a1[TB];
  uint32_t sa[TB];
  u32x4 b0[NT], b1[NT];
  uint32_t sb[NT];
};

template <int FMT, int NT, int TB>
__device__ __forceinline__ void mx_load(MxStep<FMT, NT, TB>& st, const MxArgs& a, __amdgpu_buffer_rsrc_t wq,
                                        __amdgpu_buffer_rsrc_t ws, __amdgpu_buffer_rsrc_t xq,
                                        __amdgpu_buffer_rsrc_t xs, const int (&tile)[NT], int k, int ks1,
                                        const uint32_t (&xrow)[TB], const uint32_t (&srow)[TB], int lane) {
  const int g = lane >> 4;
  const bool ok = k < ks1;
  const int col = k * 128 + 16 * g;
  // activations: K tail chunks and k-steps past the range read as zeros
  // (absent tokens have bases of 2^31 or more; OR-ing the mask keeps them there)
  const uint32_t m0 = (ok && col < a.K) ? 0u : kOOB, m1 = (ok && col + 64 < a.K) ? 0u : kOOB;
  const uint32_t ms = (ok && 4 * k + g < a.G) ? 0u : kOOB;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    st.a0[b] = ld128s(xq, (xrow[b] + (uint32_t)(16 * g)) | m0, (uint32_t)k * 128u);
    st.a1[b] = ld128s(xq, (xrow[b] + (uint32_t)(64 + 16 * g)) | m1, (uint32_t)k * 128u);
    st.sa[b] = ld8s(xs, (srow[b] + (uint32_t)g) | ms, (uint32_t)k * 4u);
  }
  const uint32_t bad = ok ? 0u : kOOB;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t tau = (uint32_t)tile[t] * (uint32_t)a.KS + (uint32_t)k;
    if constexpr (FMT == MXFP8) {
      st.b0[t] = ld128s_nt(wq, (uint32_t)lane * 16u | bad, tau * 2048u);
      st.b1[t] = ld128s_nt(wq, (1024u + (uint32_t)lane * 16u) | bad, tau * 2048u);
    } else {
      st.b0[t] = ld128s_nt(wq, (uint32_t)lane * 16u | bad, tau * 1024u);
      st.b1[t] = u32x4{0u, 0u, 0u, 0u};
    }
    st.sb[t] = ld8s(ws, (uint32_t)lane | bad, tau * 64u);
  }
}

__device__ __forceinline__ i32x8 join8(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int FMT, int NT, int TB>
__device__ __forceinline__ void mx_mma(f32x4 (&acc)[NT][TB], const MxStep<FMT, NT, TB>& st) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const i32x8 B = join8(st.b0[t], st.b1[t]);
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      // A: FP8 E4M3 (format 0); B: FP8 E4M3 (0) or FP4 E2M1 (4)
      acc[t][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(join8(st.a0[b], st.a1[b]), B, acc[t][b], 0,
                                                                   FMT == MXFP8 ? 0 : 4, 0, (int)st.sa[b], 0,
                                                                   (int)st.sb[t]);
    }
  }
}

// Workgroup = NT row tiles (SwiGLU: NT/2 gate tiles and their up tiles); its
// W waves split the k-steps; the waves' partial sums meet in LDS and are
// added in wave order (reproducible). TB blocks of 16 tokens (N <= 16 TB)
// share every weight operand: one MFMA per tile, block and k-step.
// QH (SwiGLU, two gate/up pairs = 32 columns of h): the epilogue quantises
// bf16(h) to MXFP8 exactly as qgemv_act_quant does, each 32-column block of a
// token lying inside one workgroup; h itself is stored only if y is given.
template <int FMT, int NT, bool SWIGLU, int TB, bool QH = false>
__global__ __launch_bounds__(512) void k_mxgemv(MxArgs a) {
  extern __shared__ __attribute__((aligned(16))) float red[];   // [W][NT][TB][64 lanes][4]
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane & 15;
  const __amdgpu_buffer_rsrc_t wq = make_rsrc(a.wq, a.wq_bytes);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.ws, a.ws_bytes);
  const __amdgpu_buffer_rsrc_t xq = make_rsrc(a.xq, a.xq_bytes);
  const __amdgpu_buffer_rsrc_t xs = make_rsrc(a.xs, a.xs_bytes);
  constexpr int TO = SWIGLU ? NT / 2 : NT;   // output tiles per workgroup
  static_assert(!SWIGLU || NT % 2 == 0, "SwiGLU pairs each gate tile with its up tile");
  static_assert(!QH || (SWIGLU && TO == 2), "the quantised output takes 32 columns of h per workgroup");
  int tile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int ot = min((int)blockIdx.x * TO + (SWIGLU ? t % TO : t), a.out_tiles - 1);
    tile[t] = (SWIGLU && t >= TO) ? a.up_tile0 + ot : ot;
  }
  // A row r of block b = token 16 b + r: rows past N start out of range
  uint32_t xrow[TB], srow[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int tk = 16 * b + r;
    xrow[b] = tk < a.N ? (uint32_t)(tk * a.K) : kOOB;
    srow[b] = tk < a.N ? (uint32_t)(tk * a.G) : kOOB;
  }
  f32x4 acc[NT][TB];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ks0 = wave * a.ks_per_wave;
  const int ks1 = min(a.KS, ks0 + a.ks_per_wave);
  if (ks0 < ks1) {
    // software pipeline: two k-steps in flight while one is multiplied
    MxStep<FMT, NT, TB> s0, s1, s2;
    mx_load<FMT, NT, TB>(s0, a, wq, ws, xq, xs, tile, ks0, ks1, xrow, srow, lane);
    mx_load<FMT, NT, TB>(s1, a, wq, ws, xq, xs, tile, ks0 + 1, ks1, xrow, srow, lane);
    for (int k = ks0; k < ks1; k += 3) {
      mx_load<FMT, NT, TB>(s2, a, wq, ws, xq, xs, tile, k + 2, ks1, xrow, srow, lane);
      mx_mma<FMT, NT, TB>(acc, s0);
      if (k + 1 >= ks1) break;
      mx_load<FMT, NT, TB>(s0, a, wq, ws, xq, xs, tile, k + 3, ks1, xrow, srow, lane);
      mx_mma<FMT, NT, TB>(acc, s1);
      if (k + 2 >= ks1) break;
      mx_load<FMT, NT, TB>(s1, a, wq, ws, xq, xs, tile, k + 4, ks1, xrow, srow, lane);
      mx_mma<FMT, NT, TB>(acc, s2);
    }
  }
  // lane l holds D[token 16 b + 4 (l / 16) + i][row l % 16]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < TB; ++b)
      *reinterpret_cast<f32x4*>(red + ((size_t)((wave * NT + t) * TB + b) * 64 + lane) * 4) = acc[t][b];
  __syncthreads();
  float* hb = red + (size_t)W * NT * TB * 256;   // QH: h [16 TB tokens][16 TO columns]
  for (int o = threadIdx.x; o < TO * TB * 256; o += blockDim.x) {
    const int t = o / (TB * 256), rem = o - t * TB * 256;
    const int b = rem >> 8, tl = (rem >> 4) & 15, row = rem & 15;
    const int tok = 16 * b + tl;
    const int ot = (int)blockIdx.x * TO + t;
    const int col = ot * 16 + row;
    if (!QH && (tok >= a.N || ot >= a.out_tiles || col >= a.M)) continue;
    const int idx = b * 256 + ((tl >> 2) * 16 + row) * 4 + (tl & 3);
    float v = 0.f;
    for (int w = 0; w < W; ++w) v += red[(size_t)(w * NT + t) * TB * 256 + idx];
    const size_t at = (size_t)tok * a.M + col;
    if constexpr (SWIGLU) {
      float u = 0.f;
      for (int w = 0; w < W; ++w) u += red[(size_t)(w * NT + TO + t) * TB * 256 + idx];
      v = v / (1.0f + expf(-v)) * u;
    } else {
      if (a.res) v += a.res[at];
    }
    if constexpr (QH) {
      hb[tok * (16 * TO) + t * 16 + row] = v;
      if (a.y && tok < a.N) a.y[at] = v;
    } else {
      a.y[at] = v;
    }
  }
  if constexpr (QH) {
    __syncthreads();
    // eight lanes per (token, 32-column block), four values each: the block's
    // amax over the bf16 magnitudes as integers, X = floor(log2 amax) - 8 in
    // [-127, 127], codes of bf16(h) * 2^-X (qgemv_act_quant's steps). The
    // trip count is a multiple of 64, so the eight lanes run together.
    for (int q = threadIdx.x; q < TB * 16 * 8; q += blockDim.x) {
      const int tok = q >> 3, sub = q & 7;
      const float* hv = hb + tok * 32 + sub * 4;
      uint32_t bits[4], m = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bits[i] = bf16_rne_bits(hv[i]);
        m = max(m, bits[i] & 0x7FFFu);
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 1, 8));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2, 8));
      m = max(m, (uint32_t)__shfl_xor((int)m, 4, 8));
      int X = (int)(m >> 7) - 127 - 8;
      X = m == 0 ? -127 : max(-127, min(127, X));
      const float sc = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) c |= e4m3_rne_sat(__uint_as_float(bits[i] << 16) * sc) << (8 * i);
      const int col0 = (int)blockIdx.x * 32 + sub * 4;
      if (tok < a.N && col0 < a.M) {
        *reinterpret_cast<uint32_t*>(a.hq + (size_t)tok * a.M + col0) = c;
        if (sub == 0) a.hs[(size_t)tok * (a.M / 32) + (col0 >> 5)] = (uint8_t)(X + 127);
      }
    }
  }
}

// ---- dequantisation dump ----------------------------------------------------
// One thread per (tile, k-step, lane): its 32 codes (MXFP8: two 16-code runs).
template <int FMT>
__global__ __launch_bounds__(256) void k_mx_dequant(const uint8_t* wqp, const uint8_t* wsp, int M, int K, int KS,
                                                    int RT, float* out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)RT * KS * 64) return;
  const int lane = (int)(gid & 63);
  const int64_t tau = gid >> 6;
  const int rt = (int)(tau / KS), ks = (int)(tau % KS);
  const int r = lane & 15, g = lane >> 4;
  const int row = rt * 16 + r;
  if (row >= M) return;
  const uint8_t* sc = wsp + tau * 64;
  for (int e = 0; e < 32; ++e) {
    int k;
    uint32_t code;
    if constexpr (FMT == MXFP8) {
      const int h = e >> 4, i = e & 15;
      k = 64 * h + 16 * g + i;
      code = wqp[tau * 2048 + h * 1024 + lane * 16 + i];
    } else {
      k = 32 * g + e;
      code = (wqp[tau * 1024 + lane * 16 + (e >> 1)] >> (4 * (e & 1))) & 15u;
    }
    const int kk = ks * 128 + k;
    if (kk >= K) continue;
    const int eb = sc[(k >> 5) * 16 + r];
    float v;
    if constexpr (FMT == MXFP8) {
      const int ex = (code >> 3) & 15, m = code & 7;
      v = ex ? ldexpf((float)(8 + m), ex - 10) : ldexpf((float)m, -9);
      if ((code & 0x7F) == 0x7F) v = __builtin_nanf("");
      if (code & 0x80) v = -v;
    } else {
      const float tab[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
      v = tab[code & 7];
      if (code & 8) v = -v;
    }
    out[(int64_t)row * K + kk] = eb == 255 ? __builtin_nanf("") : ldexpf(v, eb - 127);
  }
}

}  // namespace qg

// ============================================================================
// Host side
// ============================================================================
using namespace qg;

namespace {

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct MxShape {
  int nt, waves, kpw;
};

// Tiles per workgroup and k-steps per wave, from sweeps on MI355X over
// [17408][5120], [5120][17408] and [7168][5120], N = 1, 4, 8, 16, tiles per
// workgroup 1 / 2 / 4 and 8-24 k-steps per wave: MXFP8 with >= 512 tiles at
// N <= 8 takes one tile per workgroup, everything else two (two tiles halve
// how often the activations are re-read, which matters from N = 16); 8
// k-steps per wave, 16 for MXFP4 at N <= 4; fewer while the grid holds under
// ~900 waves, at most 8 waves per workgroup.
MxShape mx_shape(int fmt, int64_t out_tiles, int64_t KS, int N) {
  MxShape s;
  s.nt = (fmt == MXFP8 && out_tiles >= 512 && N <= 8) ? 1 : 2;
  const int64_t wgs = (out_tiles + s.nt - 1) / s.nt;
  int64_t kpw = (fmt == MXFP4 && N <= 4) ? 16 : 8;
  while (kpw > 1 && wgs * ((KS + kpw - 1) / kpw) < 900) --kpw;
  while ((KS + kpw - 1) / kpw > 8) ++kpw;
  s.waves = (int)((KS + kpw - 1) / kpw);
  s.kpw = (int)kpw;
  return s;
}

// SwiGLU: one gate/up pair per workgroup, the same k-steps per wave
MxShape mx_shape_pairs(int fmt, int64_t pairs, int64_t KS, int N) {
  MxShape s;
  s.nt = 2;
  int64_t kpw = (fmt == MXFP4 && N <= 4) ? 16 : 8;
  while (kpw > 1 && pairs * ((KS + kpw - 1) / kpw) < 900) --kpw;
  while ((KS + kpw - 1) / kpw > 8) ++kpw;
  s.waves = (int)((KS + kpw - 1) / kpw);
  s.kpw = (int)kpw;
  return s;
}

template <int FMT, int NT, bool SWIGLU, int TB, bool QH>
hipError_t launch_mx_tb(const MxArgs& a, const MxShape& s, hipStream_t stream) {
  const int TO = SWIGLU ? NT / 2 : NT;
  const dim3 grid((unsigned)((a.out_tiles + TO - 1) / TO));
  const dim3 block((unsigned)(64 * s.waves));
  const size_t lds = ((size_t)s.waves * NT * TB * 256 + (QH ? (size_t)TB * 16 * 16 * TO : 0)) * sizeof(float);
  hipLaunchKernelGGL((k_mxgemv<FMT, NT, SWIGLU, TB, QH>), grid, block, lds, stream, a);
  return hipGetLastError();
}

// one or two blocks of 16 tokens
template <int FMT, int NT, bool SWIGLU = false, bool QH = false>
hipError_t launch_mx(const MxArgs& a, const MxShape& s, hipStream_t stream) {
  return a.N > 16 ? launch_mx_tb<FMT, NT, SWIGLU, 2, QH>(a, s, stream)
                  : launch_mx_tb<FMT, NT, SWIGLU, 1, QH>(a, s, stream);
}

}  // namespace

int qg::mx_dequant(int fmt, const void* wq, const void* ws, int64_t M, int64_t K, float* w_out, hipStream_t stream) {
  Geom g;
  if (!geom(fmt, M, K, &g)) return QGEMV_EINVAL;
  if (g.wq_bytes >= (1ull << 31) || (uint64_t)M * (uint64_t)K >= (1ull << 40)) return QGEMV_EUNSUPPORTED;
  const int64_t threads = g.RT * g.KS * 64;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (fmt == MXFP8)
    hipLaunchKernelGGL((k_mx_dequant<MXFP8>), grid, dim3(256), 0, stream, (const uint8_t*)wq, (const uint8_t*)ws,
                       (int)M, (int)K, (int)g.KS, (int)g.RT, w_out);
  else
    hipLaunchKernelGGL((k_mx_dequant<MXFP4>), grid, dim3(256), 0, stream, (const uint8_t*)wq, (const uint8_t*)ws,
                       (int)M, (int)K, (int)g.KS, (int)g.RT, w_out);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

extern "C" int qgemv_act_quant(const void* x, int N, int64_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  if (!x || !codes || !scales) return QGEMV_EINVAL;
  if (N < 1 || K < 32) return QGEMV_EINVAL;
  if (K % 32) return QGEMV_EALIGN;
  if (!al16(x) || !al16(codes)) return QGEMV_EALIGN;
  if ((uint64_t)N * (uint64_t)K * 2ull >= (1ull << 40)) return QGEMV_EUNSUPPORTED;
  const int64_t nblk = (int64_t)N * (K / 32);
  const dim3 grid((unsigned)((nblk * 8 + 255) / 256));
  hipLaunchKernelGGL(k_act_quant, grid, dim3(256), 0, stream, (const uint16_t*)x, nblk, codes, scales);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

namespace {

// Mout output columns; Mpacked packed rows (SwiGLU: 2 Mout, gate rows first)
// hq, hs (SwiGLU only): MXFP8 codes and scales of bf16(h) instead of y
int run_mx(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs, const float* residual,
           float* y, int64_t Mout, int64_t Mpacked, int64_t K, int N, bool swiglu, hipStream_t stream,
           uint8_t* hq = nullptr, uint8_t* hs = nullptr) {
  const bool qh = hq != nullptr;
  if (fmt != MXFP8 && fmt != MXFP4) return QGEMV_EFORMAT;
  if (!wq || !ws || !xq || !xs || (!y && !qh) || (qh && (!hs || !swiglu))) return QGEMV_EINVAL;
  if (Mout < 1 || K < 32 || Mpacked > (1 << 24)) return QGEMV_EINVAL;
  if (K % 32) return QGEMV_EALIGN;
  if (N < 1 || N > 32) return QGEMV_EUNSUPPORTED;
  if (!al16(wq) || !al16(ws) || !al16(xq) || !al4(y) || (residual && !al4(residual)) || !al4(hq)) return QGEMV_EALIGN;
  if (qh && Mout % 32) return QGEMV_EALIGN;
  Geom g;
  if (!geom(fmt, Mpacked, K, &g)) return QGEMV_EINVAL;
  // k-steps past a wave's range are loaded with an out-of-range lane offset
  // (2^31 or more) on top of a tile offset up to 4 k-steps past the matrix:
  // the sum must stay below 2^32
  if (g.wq_bytes + 16384 >= (1ull << 31) || g.ws_bytes + 16384 >= (1ull << 31)) return QGEMV_EUNSUPPORTED;
  if ((uint64_t)N * (uint64_t)K >= (1ull << 30)) return QGEMV_EUNSUPPORTED;
  MxArgs a;
  a.wq = (const uint8_t*)wq;
  a.ws = (const uint8_t*)ws;
  a.xq = xq;
  a.xs = xs;
  a.res = residual;
  a.y = y;
  a.wq_bytes = (uint32_t)g.wq_bytes;
  a.ws_bytes = (uint32_t)g.ws_bytes;
  a.xq_bytes = (uint32_t)((int64_t)N * K);
  a.xs_bytes = (uint32_t)((int64_t)N * (K / 32));
  a.M = (int)Mout;
  a.K = (int)K;
  a.KS = (int)g.KS;
  a.G = (int)(K / 32);
  a.N = N;
  a.out_tiles = (int)((Mout + 15) / 16);
  a.up_tile0 = swiglu ? (int)(Mout / 16) : 0;
  a.hq = hq;
  a.hs = hs;
  MxShape s = mx_shape(fmt, a.out_tiles, g.KS, N);
  if (swiglu) s = mx_shape_pairs(fmt, a.out_tiles, g.KS, N);
  // the quantised SwiGLU's workgroups own two gate/up pairs: half the
  // k-steps per wave keeps a wave's bytes those of the plain launch (measured
  // faster for MXFP8 at every N and for MXFP4 from 8 tokens; MXFP4 at one
  // token keeps the plain split)
  if (qh && (fmt == MXFP8 || N >= 8)) {
    const int64_t kpw = std::max<int64_t>((g.KS + 7) / 8, s.kpw / 2);
    s.kpw = (int)kpw;
    s.waves = (int)((g.KS + kpw - 1) / kpw);
  }
  a.ks_per_wave = s.kpw;
  hipError_t e;
  if (qh) e = fmt == MXFP8 ? launch_mx<MXFP8, 4, true, true>(a, s, stream) : launch_mx<MXFP4, 4, true, true>(a, s, stream);
  else if (swiglu) e = fmt == MXFP8 ? launch_mx<MXFP8, 2, true>(a, s, stream) : launch_mx<MXFP4, 2, true>(a, s, stream);
  else if (fmt == MXFP8) e = s.nt == 1 ? launch_mx<MXFP8, 1>(a, s, stream) : launch_mx<MXFP8, 2>(a, s, stream);
  else e = s.nt == 1 ? launch_mx<MXFP4, 1>(a, s, stream) : launch_mx<MXFP4, 2>(a, s, stream);
  return e == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

}  // namespace

extern "C" int qgemv_mx(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs,
                        const float* residual, float* y, int64_t M, int64_t K, int N, hipStream_t stream) {
  return run_mx(fmt, wq, ws, xq, xs, residual, y, M, M, K, N, false, stream);
}

extern "C" int qgemv_mx_swiglu(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs,
                               float* h, int64_t I, int64_t K, int N, hipStream_t stream) {
  if (I < 1) return QGEMV_EINVAL;
  if (I % 16) return QGEMV_EALIGN;
  return run_mx(fmt, wq, ws, xq, xs, nullptr, h, I, 2 * I, K, N, true, stream);
}

extern "C" int qgemv_mx_swiglu_quant(int fmt, const void* wq, const void* ws, const uint8_t* xq, const uint8_t* xs,
                                     float* h, uint8_t* hq, uint8_t* hs, int64_t I, int64_t K, int N,
                                     hipStream_t stream) {
  if (!hq || !hs || I < 1) return QGEMV_EINVAL;
  if (I % 32) return QGEMV_EALIGN;
  if ((uint64_t)N * (uint64_t)I >= (1ull << 31)) return QGEMV_EUNSUPPORTED;
  return run_mx(fmt, wq, ws, xq, xs, nullptr, h, I, 2 * I, K, N, true, stream, hq, hs);
}
