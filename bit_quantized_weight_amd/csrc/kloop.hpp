// The weight-streaming inner loop shared by the dense and MoE kernels.
//
// One wave owns NT row tiles (16 weight rows each) and a range of k-steps
// (128 columns = 4 scale groups). Per k-step and tile it issues one 16-byte
// non-temporal load per lane for the codes (int8: two), plus the scale
// record (and the int5 hi-bit word), decodes each group into the B operand of
// a 16x16x32 bf16 MFMA and accumulates in fp32 per tile.
//
// A operand rows are (slot, token) = 8 * slot + token. The caller's ALoad
// functor returns this lane's 8 activations of a group (bf16x8) and must
// return zeros when `use` is false; the slot roles are:
//   int formats: group j of a k-step lives in slot j & 1, so one accumulator
//     holds two groups apart and the scale step runs per pair of groups;
//   nvfp4: the two 16-column blocks of a group live in slots 0 and 1
//     (lanes with s = lane/16 in {0,1} hold block 0, {2,3} block 1).
// After the loop, lane l's acc[t][i] is the partial sum of A row 4*(l/16) + i
// for weight row 16*tile + (l % 16) (NVFP4 without the tensor scale).
#pragma once
#include "device.hpp"
#include "layout.hpp"

namespace qg {

template <int FMT>
__device__ __forceinline__ void group_pair_scale(f32x4& acc, const f32x4& D, const f32x4& Db, uint32_t sc) {
  if constexpr (FMT == INT8) {
    const float d = f16_lo(sc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(d, D[i], acc[i]);
  } else {
    // D = sum x (128 + q), Db = 128 sum x:  d*sum(x q) + m*sum(x) = d*D + (m/128 - d)*Db
    const float d = f16_lo(sc), m = f16_hi(sc);
    const float c = fmaf(m, 0.0078125f, -d);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = fmaf(d, D[i], acc[i]);
      acc[i] = fmaf(c, Db[i], acc[i]);
    }
  }
}

// true when this lane's A row takes part in group j (see header comment)
template <int FMT>
__device__ __forceinline__ bool a_slot_uses(int a_slot, int s, int j) {
  return FMT == NVFP4 ? (a_slot == (s >> 1)) : (a_slot == (j & 1));
}

template <int FMT, int NT, class ALoad>
__device__ __forceinline__ void kloop(__amdgpu_buffer_rsrc_t wq, __amdgpu_buffer_rsrc_t ws, const int (&tile)[NT],
                                      int KS, int ks0, int ks1, uint32_t hi_offset, const ALoad& aload,
                                      f32x4 (&acc)[NT]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, s = lane >> 4;
  const int a_slot = r >> 3;
  const bf16x8 b128 = bf16x8_splat_128();

  for (int ks = ks0; ks < ks1; ++ks) {
    u32x4 cw[NT], cw2[NT];
    uint32_t hw[NT], sc32[NT];
    u32x2 sc64[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t tau = (uint32_t)tile[t] * (uint32_t)KS + (uint32_t)ks;
      if constexpr (FMT == INT8) {
        cw[t] = ld128_nt(wq, tau * 2048u + (uint32_t)lane * 16u);
        cw2[t] = ld128_nt(wq, tau * 2048u + 1024u + (uint32_t)lane * 16u);
        sc32[t] = ld32(ws, tau * 128u + (uint32_t)r * 8u + 4u * (uint32_t)(s >> 1));
      } else if constexpr (FMT == NVFP4) {
        cw[t] = ld128_nt(wq, tau * 1024u + (uint32_t)lane * 16u);
        sc32[t] = ld32(ws, tau * 128u + (uint32_t)r * 8u + 4u * (uint32_t)(s >> 1));
      } else {
        cw[t] = ld128_nt(wq, tau * 1024u + (uint32_t)lane * 16u);
        if constexpr (FMT == INT5)
          hw[t] = __builtin_amdgcn_raw_buffer_load_b32(wq, hi_offset + tau * 256u + (uint32_t)lane * 4u, 0,
                                                       kNonTemporal);
        sc64[t] = ld64(ws, tau * 256u + (uint32_t)r * 16u + 8u * (uint32_t)(s >> 1));
      }
    }
    bf16x8 A[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) A[j] = aload(ks, j, a_slot_uses<FMT>(a_slot, s, j));

    if constexpr (FMT == NVFP4) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t v = j == 0 ? cw[t].x : j == 1 ? cw[t].y : j == 2 ? cw[t].z : cw[t].w;
          const f32x4 D = mfma(A[j], dec_nvfp4(v), f32x4{0.f, 0.f, 0.f, 0.f});
          float sc;
          if (j == 0) sc = e4m3_byte<0>(sc32[t]);
          else if (j == 1) sc = e4m3_byte<1>(sc32[t]);
          else if (j == 2) sc = e4m3_byte<2>(sc32[t]);
          else sc = e4m3_byte<3>(sc32[t]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(sc, D[i], acc[t][i]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x4 Db = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT != INT8) {
          Db = mfma(A[2 * c], b128, Db);
          Db = mfma(A[2 * c + 1], b128, Db);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          bf16x8 B0, B1;
          if constexpr (FMT == INT4) {
            B0 = dec_int4(c == 0 ? cw[t].x : cw[t].z);
            B1 = dec_int4(c == 0 ? cw[t].y : cw[t].w);
          } else if constexpr (FMT == INT5) {
            if (c == 0) {
              B0 = dec_int5<0>(cw[t].x, hw[t]);
              B1 = dec_int5<1>(cw[t].y, hw[t]);
            } else {
              B0 = dec_int5<2>(cw[t].z, hw[t]);
              B1 = dec_int5<3>(cw[t].w, hw[t]);
            }
          } else {  // INT8: groups 0,1 in the first 1 KiB, 2,3 in the second
            const u32x4 q = c == 0 ? cw[t] : cw2[t];
            B0 = dec_int8(q.x, q.y);
            B1 = dec_int8(q.z, q.w);
          }
          f32x4 D = mfma(A[2 * c], B0, f32x4{0.f, 0.f, 0.f, 0.f});
          D = mfma(A[2 * c + 1], B1, D);
          uint32_t sc;
          if constexpr (FMT == INT8) sc = c == 0 ? (sc32[t] & 0xFFFFu) : (sc32[t] >> 16);
          else sc = c == 0 ? sc64[t].x : sc64[t].y;
          group_pair_scale<FMT>(acc[t], D, Db, sc);
        }
      }
    }
  }
}

}  // namespace qg
