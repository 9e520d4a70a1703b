// Host-side quantiser and packer (qgemv_pack, qgemv_pack_codes).
//
// Formats per the NInfer article (section 2: groupwise Q4/Q5 integers and
// NVFP4 weights), the RustingStrata page (Q8_0-style int8) and the Decapybara
// page (NVFP4 with E4M3 block scales). The pages give no quantisation rule;
// the rules here are the plainest readings, stated in include/qgemv.h.
//
// Floating-point steps happen in the stated precision, in source order, with
// FMA contraction disabled for this file (-ffp-contract=off): fp32 for the
// scale arithmetic, fp64 for the code division, one round-to-nearest-even for
// every conversion. That makes the bytes reproducible on any IEEE host.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "layout.hpp"
#include "qgemv.h"

namespace {

using qg::Geom;

// ---- encodings -----------------------------------------------------------

// IEEE binary32 -> binary16, round to nearest, ties to even; overflow -> inf.
uint16_t f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds past 65504
  const uint32_t e = a >> 23;
  if (e < 113) {  // below 2^-14: fp16 subnormal (or zero), units of 2^-24
    if (e == 0) return (uint16_t)sign;  // fp32 subnormal: far below 2^-25
    const uint32_t m = (a & 0x7FFFFFu) | 0x800000u;  // value = m * 2^(e-150)
    const int sh = 126 - (int)e;                      // n = m / 2^sh
    if (sh > 24) return (uint16_t)sign;
    uint32_t n = m >> sh;
    const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
    if (rem > half || (rem == half && (n & 1u))) ++n;
    return (uint16_t)(sign | n);
  }
  uint32_t r = ((e - 112u) << 10) | ((a & 0x7FFFFFu) >> 13);
  const uint32_t rem = a & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  return (uint16_t)(sign | r);
}

double f16_to_f64(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

bool f16_is_finite(uint16_t h) { return ((h >> 10) & 0x1F) != 0x1F; }

// OCP FP8 E4M3 value of a code (NaN for S.1111.111).
double e4m3_to_f64(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e ? ldexp((double)(8 + m), e - 10) : ldexp((double)m, -9);
  return s ? -v : v;
}

// Non-negative fp32 -> E4M3 code, nearest-even, saturating at 448.
uint8_t e4m3_from_f32(float f) {
  const double v = (double)f;
  if (!(v > 0)) return 0;
  if (v >= 448.0) return 0x7E;
  if (v < 0.015625) {  // below 2^-6: subnormal steps of 2^-9 (8 -> 2^-6, code 8)
    return (uint8_t)nearbyint(v * 512.0);
  }
  int e;
  const double fr = frexp(v, &e);  // v = fr * 2^e, fr in [0.5, 1)
  const double mant = fr * 2.0;    // [1, 2), exponent e - 1
  const int n = (int)nearbyint((mant - 1.0) * 8.0);
  int code = ((e - 1 + 7) << 3) + n;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)code;
}

// E4M3 code for a double, nearest-even, saturating at +-448; sign bit = sign of v.
uint8_t e4m3_from_f64_signed(double v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0;
  const double a = fabs(v);
  uint8_t mag;
  if (a >= 448.0) {
    mag = 0x7E;
  } else if (a < 0.015625) {               // subnormal steps of 2^-9 (8 -> least normal, code 8)
    mag = (uint8_t)nearbyint(a * 512.0);
  } else {
    int e;
    const double fr = frexp(a, &e);        // a = fr * 2^e, fr in [0.5, 1)
    const int n = (int)nearbyint((fr * 2.0 - 1.0) * 8.0);
    mag = (uint8_t)std::min(0x7E, ((e - 1 + 7) << 3) + n);
  }
  return (uint8_t)(mag | sign);
}

// MX block scale exponent: floor(log2(amax)) - emax clamped to [-127, 127];
// -127 for an all-zero block.
int mx_exponent(double amax, int emax) {
  if (amax == 0.0) return -127;
  int p;
  frexp(amax, &p);                          // amax = f * 2^p, f in [0.5, 1)
  return std::max(-127, std::min(127, p - 1 - emax));
}

// E2M1 code for a double, nearest-even, saturating at +-6; sign bit = sign of v.
uint8_t e2m1_from_f64(double v) {
  const uint8_t sign = signbit(v) ? 8 : 0;
  const double a = fabs(v);
  uint8_t mag;
  if (a >= 6.0) mag = 7;
  else if (a < 1.0) mag = (uint8_t)nearbyint(a * 2.0);                       // 0, 0.5, 1.0
  else if (a < 2.0) mag = (uint8_t)(2 + (int)nearbyint((a - 1.0) * 2.0));    // 1, 1.5, 2
  else if (a < 4.0) mag = (uint8_t)(4 + (int)nearbyint((a * 0.5 - 1.0) * 2.0));
  else mag = (uint8_t)(6 + (int)nearbyint((a * 0.25 - 1.0) * 2.0));         // 4, 6
  return (uint8_t)(mag | sign);
}

// ---- scatter into the layout ----------------------------------------------

struct Dest {
  const Geom* g;
  int fmt;
  uint8_t* wq;
  uint8_t* ws;
  // one column k of row m gets code c
  inline void code(int64_t m, int64_t k, int c) const {
    const int64_t rt = m >> 4, r = m & 15, ks = k >> 7, j = (k >> 5) & 3, s = (k >> 3) & 3, e = k & 7;
    const int64_t tau = rt * g->KS + ks, lane = s * 16 + r;
    if (fmt == qg::INT8) {
      wq[tau * 2048 + (j >> 1) * 1024 + lane * 16 + (j & 1) * 8 + e] = (uint8_t)(int8_t)c;
      return;
    }
    if (fmt == qg::MXFP8 || fmt == qg::MXFP4) {
      const int64_t kk = k & 127;
      if (fmt == qg::MXFP8) {
        const int64_t h = kk >> 6, gg = (kk >> 4) & 3, i = kk & 15;
        wq[tau * 2048 + h * 1024 + (gg * 16 + r) * 16 + i] = (uint8_t)c;
      } else {
        const int64_t gg = kk >> 5, i = (kk & 31) >> 1, sh = 4 * (kk & 1);
        uint8_t* p = wq + tau * 1024 + (gg * 16 + r) * 16 + i;
        *p = (uint8_t)(*p | ((c & 15) << sh));
      }
      return;
    }
    if (fmt == qg::INT5) {  // 5-bit fields, three pairs per dword; pair 15 spread over bit 15/31
      const int64_t P = 4 * j + (e >> 1), h = e & 1;
      if (P < 15) {
        or_dword(int5_dword(tau, lane, (int)(P / 3)), (uint32_t)(c & 31) << (16 * h + 5 * (P % 3)));
      } else {
        for (int b = 0; b < 5; ++b)
          if ((c >> b) & 1) or_dword(int5_dword(tau, lane, b), 1u << (16 * h + 15));
      }
      return;
    }
    int64_t byte, shift;
    if (fmt == qg::NVFP4) {
      byte = tau * 1024 + lane * 16 + 4 * j + (e >> 1);
      shift = 4 * (e & 1);
    } else {
      const int64_t i = (e & 1) ? 4 + (e >> 1) : (e >> 1);
      byte = tau * 1024 + lane * 16 + 4 * j + (i >> 1);
      shift = 4 * (i & 1);
    }
    wq[byte] = (uint8_t)(wq[byte] | ((c & 15) << shift));
  }
  // int5: dwords 0..3 of a lane in plane A, dword 4 in plane B
  inline uint8_t* int5_dword(int64_t tau, int64_t lane, int i) const {
    return i < 4 ? wq + tau * 1024 + lane * 16 + 4 * i : wq + g->hi_offset + tau * 256 + lane * 4;
  }
  static inline void or_dword(uint8_t* p, uint32_t v) {
    for (int b = 0; b < 4; ++b) p[b] = (uint8_t)(p[b] | (v >> (8 * b)));
  }
  // per-group scale fields (int formats), group index gi along K
  inline void group(int64_t m, int64_t gi, uint16_t d, uint16_t mn) const {
    const int64_t rt = m >> 4, r = m & 15, ks = gi >> 2, j = gi & 3;
    const int64_t tau = rt * g->KS + ks, pos = qg::scale_pos((int)j);
    if (fmt == qg::INT8) {
      uint8_t* p = ws + tau * 128 + r * 8 + 2 * pos;
      p[0] = (uint8_t)d;
      p[1] = (uint8_t)(d >> 8);
    } else {
      uint8_t* p = ws + tau * 256 + r * 16 + 4 * pos;
      p[0] = (uint8_t)d;
      p[1] = (uint8_t)(d >> 8);
      p[2] = (uint8_t)mn;
      p[3] = (uint8_t)(mn >> 8);
    }
  }
  // NVFP4 block scale, block index bi along K (16 columns each)
  inline void block(int64_t m, int64_t bi, uint8_t sb) const {
    const int64_t rt = m >> 4, r = m & 15, ks = bi >> 3, j = (bi >> 1) & 3, h = bi & 1;
    ws[(rt * g->KS + ks) * 128 + r * 8 + 4 * h + j] = sb;
  }
  inline void tensor_scale(float st) const { memcpy(ws + g->st_offset, &st, 4); }
  // MX E8M0 scale of 32-block bi along K
  inline void mx_scale(int64_t m, int64_t bi, uint8_t e) const {
    const int64_t rt = m >> 4, r = m & 15, ks = bi >> 2, gg = bi & 3;
    ws[(rt * g->KS + ks) * 64 + gg * 16 + r] = e;
  }
};

// Runs f(row_begin, row_end) over row ranges aligned to 16 on a few threads.
// Rows of one 16-row tile stay on one thread: they share bytes of the layout.
template <class F>
void parallel_rows(int64_t M, F f) {
  const int64_t tiles = (M + 15) / 16;
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = std::min<int64_t>(hw ? hw : 1, 16);
  if (tiles < 64) nt = 1;
  nt = std::min(nt, tiles);
  if (nt <= 1) {
    f(0, M);
    return;
  }
  std::vector<std::thread> th;
  const int64_t per = (tiles + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t b = std::min(M, t * per * 16), e = std::min(M, (t + 1) * per * 16);
    if (b < e) th.emplace_back(f, b, e);
  }
  for (auto& x : th) x.join();
}

int quantize_rows(const Dest& D, const float* W, int64_t M, int64_t K) {
  const int fmt = D.fmt;
  if (fmt == qg::NVFP4) {
    float amax = 0.0f;
    for (int64_t i = 0; i < M * K; ++i) amax = std::max(amax, fabsf(W[i] + 0.0f));
    float st = amax / 2688.0f;
    if (st == 0.0f) st = 1.0f;
    D.tensor_scale(st);
    const float denom = 6.0f * st;
    parallel_rows(M, [&](int64_t m0, int64_t m1) {
      for (int64_t m = m0; m < m1; ++m) {
        const float* row = W + m * K;
        for (int64_t b = 0; b < K / 16; ++b) {
          float ab = 0.0f;
          for (int i = 0; i < 16; ++i) ab = std::max(ab, fabsf(row[b * 16 + i] + 0.0f));
          const float ratio = ab / denom;
          const uint8_t sb = e4m3_from_f32(ratio);
          D.block(m, b, sb);
          const double sbv = e4m3_to_f64(sb);
          for (int i = 0; i < 16; ++i) {
            const double w = (double)(row[b * 16 + i] + 0.0f);
            const uint8_t c = sbv == 0.0 ? 0 : e2m1_from_f64(w / (sbv * (double)st));
            D.code(m, b * 16 + i, c);
          }
        }
      }
    });
    return QGEMV_OK;
  }
  if (fmt == qg::MXFP8 || fmt == qg::MXFP4) {
    const int emax = fmt == qg::MXFP8 ? 8 : 2;
    parallel_rows(M, [&](int64_t m0, int64_t m1) {
      for (int64_t m = m0; m < m1; ++m) {
        const float* row = W + m * K;
        for (int64_t b = 0; b < K / 32; ++b) {
          double amax = 0.0;
          for (int i = 0; i < 32; ++i) amax = std::max(amax, (double)fabsf(row[b * 32 + i]));
          const int X = mx_exponent(amax, emax);
          D.mx_scale(m, b, (uint8_t)(X + 127));
          for (int i = 0; i < 32; ++i) {
            const double t = ldexp((double)(row[b * 32 + i] + 0.0f), -X);   // exact
            D.code(m, b * 32 + i, fmt == qg::MXFP8 ? e4m3_from_f64_signed(t) : e2m1_from_f64(t));
          }
        }
      }
    });
    return QGEMV_OK;
  }
  std::atomic<int> status{QGEMV_OK};
  parallel_rows(M, [&](int64_t m0, int64_t m1) {
    for (int64_t m = m0; m < m1; ++m) {
      const float* row = W + m * K;
      for (int64_t gi = 0; gi < K / 32; ++gi) {
        float v[32];
        for (int i = 0; i < 32; ++i) v[i] = row[gi * 32 + i] + 0.0f;  // -0 -> +0
        if (fmt == qg::INT8) {
          float amax = 0.0f;
          for (int i = 0; i < 32; ++i) amax = std::max(amax, fabsf(v[i]));
          const float d32 = amax / 127.0f;
          const uint16_t d16 = f32_to_f16(d32);
          if (!f16_is_finite(d16)) { status = QGEMV_ERANGE; return; }
          const double dd = f16_to_f64(d16);
          D.group(m, gi, d16, 0);
          for (int i = 0; i < 32; ++i) {
            int q = 0;
            if (dd != 0.0) {
              const double t = nearbyint((double)v[i] / dd);
              q = (int)std::min(127.0, std::max(-127.0, t));
            }
            D.code(m, gi * 32 + i, q);
          }
        } else {
          const int qmax = fmt == qg::INT4 ? 15 : 31;
          float mn = v[0], mx = v[0];
          for (int i = 1; i < 32; ++i) { mn = std::min(mn, v[i]); mx = std::max(mx, v[i]); }
          const float d32 = (mx - mn) / (float)qmax;
          const uint16_t d16 = f32_to_f16(d32), m16 = f32_to_f16(mn);
          if (!f16_is_finite(d16) || !f16_is_finite(m16)) { status = QGEMV_ERANGE; return; }
          const double dd = f16_to_f64(d16), mm = f16_to_f64(m16);
          D.group(m, gi, d16, m16);
          for (int i = 0; i < 32; ++i) {
            int q = 0;
            if (dd != 0.0) {
              const double t = nearbyint(((double)v[i] - mm) / dd);
              q = (int)std::min((double)qmax, std::max(0.0, t));
            }
            D.code(m, gi * 32 + i, q);
          }
        }
      }
    }
  });
  return status.load();
}

}  // namespace

extern "C" int qgemv_packed_bytes(int fmt, int64_t M, int64_t K, size_t* wq_bytes, size_t* ws_bytes) {
  if (fmt < qg::INT4 || fmt > qg::MXFP8) return QGEMV_EFORMAT;
  if (!wq_bytes || !ws_bytes) return QGEMV_EINVAL;
  Geom g;
  if (!qg::geom(fmt, M, K, &g)) return QGEMV_EINVAL;
  *wq_bytes = g.wq_bytes;
  *ws_bytes = g.ws_bytes;
  return QGEMV_OK;
}

extern "C" int qgemv_expert_stride(int fmt, int64_t M, int64_t K, size_t* wq_stride, size_t* ws_stride) {
  size_t a, b;
  const int rc = qgemv_packed_bytes(fmt, M, K, &a, &b);
  if (rc) return rc;
  if (!wq_stride || !ws_stride) return QGEMV_EINVAL;
  *wq_stride = (a + 255) / 256 * 256;
  *ws_stride = (b + 255) / 256 * 256;
  return QGEMV_OK;
}

extern "C" int qgemv_pack(int fmt, const float* W, int64_t M, int64_t K, void* wq, void* ws) {
  if (fmt < qg::INT4 || fmt > qg::MXFP8) return QGEMV_EFORMAT;
  if (!W || !wq || !ws) return QGEMV_EINVAL;
  Geom g;
  if (!qg::geom(fmt, M, K, &g)) return QGEMV_EINVAL;
  for (int64_t i = 0; i < M * K; ++i)
    if (!isfinite(W[i])) return QGEMV_EINVAL;
  memset(wq, 0, g.wq_bytes);
  memset(ws, 0, g.ws_bytes);
  Dest D{&g, fmt, (uint8_t*)wq, (uint8_t*)ws};
  return quantize_rows(D, W, M, K);
}

extern "C" int qgemv_pack_codes(int fmt, const void* codes, const void* scales, const uint16_t* mins,
                                float tensor_scale, int64_t M, int64_t K, void* wq, void* ws) {
  if (fmt < qg::INT4 || fmt > qg::MXFP8) return QGEMV_EFORMAT;
  if (!codes || !scales || !wq || !ws) return QGEMV_EINVAL;
  if ((fmt == qg::INT4 || fmt == qg::INT5) && !mins) return QGEMV_EINVAL;
  Geom g;
  if (!qg::geom(fmt, M, K, &g)) return QGEMV_EINVAL;
  const int lo = fmt == qg::INT8 ? -128 : 0;
  const int hi = fmt == qg::INT8 ? 127 : (fmt == qg::INT5 ? 31 : (fmt == qg::MXFP8 ? 255 : 15));
  for (int64_t i = 0; i < M * K; ++i) {
    const int c = fmt == qg::INT8 ? (int)((const int8_t*)codes)[i] : (int)((const uint8_t*)codes)[i];
    if (c < lo || c > hi) return QGEMV_EINVAL;
    if (fmt == qg::MXFP8 && (c & 0x7F) == 0x7F) return QGEMV_EINVAL;   // E4M3 NaN
  }
  if (fmt == qg::MXFP8 || fmt == qg::MXFP4) {
    const uint8_t* e = (const uint8_t*)scales;
    for (int64_t i = 0; i < M * (K / 32); ++i)
      if (e[i] == 0xFF) return QGEMV_EINVAL;                           // E8M0 NaN
  }
  memset(wq, 0, g.wq_bytes);
  memset(ws, 0, g.ws_bytes);
  Dest D{&g, fmt, (uint8_t*)wq, (uint8_t*)ws};
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) {
      const int c = fmt == qg::INT8 ? (int)((const int8_t*)codes)[m * K + k] : (int)((const uint8_t*)codes)[m * K + k];
      D.code(m, k, c);
    }
  if (fmt == qg::NVFP4) {
    const uint8_t* sb = (const uint8_t*)scales;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t b = 0; b < K / 16; ++b) D.block(m, b, sb[m * (K / 16) + b]);
    D.tensor_scale(tensor_scale);
  } else if (fmt == qg::MXFP8 || fmt == qg::MXFP4) {
    const uint8_t* e = (const uint8_t*)scales;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t b = 0; b < K / 32; ++b) D.mx_scale(m, b, e[m * (K / 32) + b]);
  } else {
    const uint16_t* d = (const uint16_t*)scales;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t gi = 0; gi < K / 32; ++gi)
        D.group(m, gi, d[m * (K / 32) + gi], mins ? mins[m * (K / 32) + gi] : 0);
  }
  return QGEMV_OK;
}
