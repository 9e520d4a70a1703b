// The weight-streaming inner loop shared by the dense and MoE kernels.
//
// One wave owns NT row tiles (16 weight rows each) and a range of k-steps
// (128 columns = 4 groups of 32). Per k-step and tile it issues one 16-byte
// non-temporal buffer load per lane for the codes (int8: two, int5: plus one
// dword), decodes each 32-column group into the B operand of a 16x16x32 bf16
// MFMA and accumulates in fp32. Loads for later k-steps are issued before the
// decode and MFMAs of k-step i: weights in two buffers of KPS k-steps, so a
// wave keeps KPS k-steps of weights in flight while it computes, and
// activations one k-step ahead. Wave-uniform offsets travel in SGPRs (buffer
// soffset); the per-lane offsets are loop constants.
//
// Slots. A operand row m (0..15) = slot * T + token with T = 16 / S tokens per
// slot. Consecutive scale units (int: 32-column groups; nvfp4: 16-column
// blocks) go to consecutive slots, so one accumulator keeps S units apart and
// the per-unit scale step runs once per S units ("cycle") instead of once per
// unit. S = 16 at N = 1, 8 at N = 2, 4 at N <= 4, 2 at N <= 8, 1 at N <= 16,
// where every group runs its own scale step (nvfp4: each of a group's two
// blocks, through an MFMA of its own, see HALVES). A lane whose
// row is not in a unit's slot gets its offset moved by the slot difference
// times 2^25 (activations stay below 2^25 bytes), so the buffer range check
// returns zeros without a memory access. Rows of absent tokens start at
// 2^30, and k-steps past the range or groups past K add 2^31: in every case
// the offset lands at least 2^25 away from [0, 2^25).
//
// Int group scale: B = bf16(c + q) with the code bias c = 16 (int4) or 32
// (int5); with D = sum x (c + q) and Db = c sum x (an MFMA against a
// constant-c operand shared by all tiles),
//   d * sum(x q) + m * sum(x) = (m / c) * Db + d * (D - Db),
// added to the accumulator in that order. Both MFMA sums carry rounding of
// order 2^-24 c sum|x|, so the error of the step grows with c d sum|x|; the
// smallest exact bias keeps it small, and forming D - Db before scaling by d
// (instead of adding d * D and subtracting d * Db) avoids a rounding at the
// magnitude of d * D. With a one-hot x of value 1 every sum is exact and the
// step gives RN(d q + m), the dequantised weight itself.
//
// After the loop, lane l's acc[t][i] is the partial sum of A row 4*(l/16) + i
// for weight row 16*tile[t] + (l % 16) (nvfp4: without the tensor scale).
#pragma once
#include "device.hpp"
#include "layout.hpp"

namespace qg {

constexpr uint32_t kSlotStride = 1u << 25;   // offset step per slot mismatch
constexpr uint32_t kAbsentRow = 1u << 30;    // lane base of an A row with no token

// ---- compile-time geometry of a (format, slots) pair
template <int FMT, int S>
struct Cyc {
  static constexpr int T = 16 / S;                          // tokens per slot
  static constexpr int UNITS_PER_GROUP = FMT == NVFP4 ? 2 : 1;
  // nvfp4 with one slot: the two 16-column blocks of a group share the slot,
  // so each block takes its own MFMA with the other block's activation lanes
  // masked to zero, and its own scale step
  static constexpr bool HALVES = FMT == NVFP4 && S == 1;
  static constexpr int GROUPS = HALVES ? 1 : S / UNITS_PER_GROUP;   // groups per cycle (>= 1)
  static_assert(GROUPS >= 1, "slots per group");
  static constexpr int KSTEPS = GROUPS >= 4 ? GROUPS / 4 : 1;   // k-steps per cycle
  static constexpr int UNROLL = KSTEPS >= 2 ? KSTEPS : 2;   // k-steps per loop trip (even)
};

// Slot of A rows that group j of k-step kk (counted from the cycle start)
// feeds; for nvfp4 the lane's block half is folded into the lane base.
template <int FMT, int S>
__host__ __device__ constexpr int slot_pos(int kk, int j) {
  return FMT == NVFP4 ? (8 * kk + 2 * j) % S : (4 * kk + j) % S;
}

// Per-lane A base offset term: (slot of this lane's row, nvfp4 minus its
// block half) * 2^25; the loader adds the row offset and subtracts
// slot_pos * 2^25, so only lanes of the unit's slot stay in range.
template <int FMT, int S>
__device__ __forceinline__ uint32_t lane_slot_term(int lane) {
  const int r = lane & 15, s = lane >> 4;
  const int sigma = r / Cyc<FMT, S>::T - ((FMT == NVFP4 && S > 1) ? (s >> 1) : 0);
  return (uint32_t)sigma * kSlotStride;
}

// ---- packed weights of KPS consecutive k-steps (all tiles)
template <int FMT, int NT, int KPS>
struct Step {
  u32x4 q[KPS][NT];      // codes: int4/nvfp4 dword j = group j; int5 dwords D0..D3; int8 groups 0,1
  u32x4 q2[KPS][NT];     // int8 groups 2,3
  uint32_t h[KPS][NT];   // int5 dword D4
  u32x4 sc[KPS][NT];     // scale words (cycles of at most one k-step)
  u32x4 cyc[NT];         // scale words of the cycle starting at this buffer (cycles of several k-steps)
};

// Scale words of one tile for the cycle whose first k-step is tile record
// tau0 (int formats: 16 B (int4/5) or 8 B (int8) records per row and k-step;
// nvfp4: 8 B of E4M3 block scales per row and k-step). krem: k-steps of the
// wave's range left from the cycle start; records past it read as zero.
// tau0 stays below 2^31 / 256 (validated), so offsets never wrap.
template <int FMT, int S>
__device__ __forceinline__ u32x4 load_scales(__amdgpu_buffer_rsrc_t ws, uint32_t tau0, int lane, int krem) {
  const int r = lane & 15, s = lane >> 4;
  u32x4 v = {0u, 0u, 0u, 0u};
  constexpr bool REC_S = FMT != NVFP4 && S == 16;                                   // record k-step s
  constexpr bool REC_S2 = (FMT != NVFP4 && S == 8) || (FMT == NVFP4 && S == 16);     // record k-step s >> 1
  const int rec = REC_S ? s : (REC_S2 ? (s >> 1) : 0);
  const uint32_t mask = rec < krem ? 0u : 0x80000000u;
  if constexpr (FMT == INT4 || FMT == INT5) {
    const uint32_t so = tau0 * 256u;
    const uint32_t row = (uint32_t)r * 16u | mask;
    if constexpr (S == 16) {          // groups 16c + 4s + i: record of k-step 4c + s, all four
      v = ld128s(ws, row + (uint32_t)s * 256u, so);
    } else if constexpr (S == 1) {    // every lane: the four groups of its row's record, pos order
      v = ld128s(ws, row, so);
    } else if constexpr (S == 8) {    // groups 8c + 2s + (i>>1): record 2c + (s>>1), j = 2(s&1) + (i>>1)
      const uint32_t b = row + (uint32_t)(s >> 1) * 256u;
      v.x = ld32s(ws, b + 4u * (uint32_t)(s & 1), so);          // pos(j) = s & 1 for i < 2
      v.y = ld32s(ws, b + 4u * (uint32_t)(2 + (s & 1)), so);    // pos(j) = 2 + (s & 1)
    } else if constexpr (S == 4) {    // group 4c + s: j = s
      v.x = ld32s(ws, row + 4u * (uint32_t)(2 * (s & 1) + (s >> 1)), so);
    } else {                          // S = 2: groups 2c + (s>>1), c = 0, 1: positions 2(s>>1) + c
      const u32x2 t = ld64s(ws, row + 8u * (uint32_t)(s >> 1), so);
      v.x = t.x;
      v.y = t.y;
    }
  } else if constexpr (FMT == INT8) {
    const uint32_t so = tau0 * 128u;
    const uint32_t row = (uint32_t)r * 8u | mask;
    if constexpr (S == 16) {
      const u32x2 t = ld64s(ws, row + (uint32_t)s * 128u, so);
      v.x = t.x;
      v.y = t.y;
    } else if constexpr (S == 1) {    // the row's four fp16 scales, pos order
      const u32x2 t = ld64s(ws, row, so);
      v.x = t.x;
      v.y = t.y;
    } else if constexpr (S == 8) {
      const u32x2 t = ld64s(ws, row + (uint32_t)(s >> 1) * 128u, so);
      const uint32_t sh = 16u * (uint32_t)(s & 1);
      v.x = t.x >> sh;   // pos s&1      -> low half
      v.y = t.y >> sh;   // pos 2 + s&1  -> low half
    } else if constexpr (S == 4) {
      v.x = ld16s(ws, row + 2u * (uint32_t)(2 * (s & 1) + (s >> 1)), so);
    } else {
      v.x = ld32s(ws, row + 4u * (uint32_t)(s >> 1), so);
    }
  } else {  // NVFP4: byte 4h + j of the row record holds block 8ks + 2j + h
    const uint32_t so = tau0 * 128u;
    const uint32_t row = (uint32_t)r * 8u | mask;
    if constexpr (S == 16) {          // blocks 16c + 4s + i: record 2c + (s>>1)
      const u32x2 t = ld64s(ws, row + (uint32_t)(s >> 1) * 128u, so);
      const uint32_t sh = 16u * (uint32_t)(s & 1);
      v.x = t.x >> sh;   // i = 0: byte 0, i = 2: byte 1 (h = 0)
      v.y = t.y >> sh;   // i = 1: byte 0, i = 3: byte 1 (h = 1)
    } else if constexpr (S == 8) {    // block 2s + (i>>1) of the k-step: j = s, h = i >> 1
      const u32x2 t = ld64s(ws, row, so);
      const uint32_t sh = 8u * (uint32_t)s;
      v.x = t.x >> sh;
      v.y = t.y >> sh;
    } else if constexpr (S == 4) {    // block 4c + s: j = 2c + (s>>1), h = s & 1
      v.x = ld32s(ws, row + 4u * (uint32_t)(s & 1), so) >> (8u * (uint32_t)(s >> 1));
    } else if constexpr (S == 1) {    // every lane: its row's whole record (x: h = 0, y: h = 1; byte j)
      const u32x2 t = ld64s(ws, row, so);
      v.x = t.x;
      v.y = t.y;
    } else {                          // S = 2: block 2j + (s>>1)
      v.x = ld32s(ws, row + 4u * (uint32_t)(s >> 1), so);
    }
  }
  return v;
}

// ---- int5: 16 pair-words (bf16x2 of 32 + q) from the lane's five dwords;
// the 5-bit code lands in mantissa bits 2..6 (one ulp of 32 is 1/4)
__device__ __forceinline__ void dec_int5_step(const u32x4& q, uint32_t d4, bf16x8 (&B)[4]) {
  const uint32_t D[5] = {q.x, q.y, q.z, q.w, d4};
  uint32_t P[16];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    P[3 * i + 0] = and_or(D[i] << 2, 0x007C007Cu, kBias5Bits);
    P[3 * i + 1] = and_or(D[i] >> 3, 0x007C007Cu, kBias5Bits);
    P[3 * i + 2] = and_or(D[i] >> 8, 0x007C007Cu, kBias5Bits);
  }
  // the 16th pair: code bit b is bit 15 (low half) / 31 (high half) of dword b
  uint32_t p15 = kBias5Bits;
#pragma unroll
  for (int b = 0; b < 5; ++b) p15 = and_or(D[b] >> (13 - b), 0x00010001u << (b + 2), p15);
  P[15] = p15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = {P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3]};
    B[j] = __builtin_bit_cast(bf16x8, v);
  }
}

// E4M3 byte j (0..3, unrolled) of a scale word
__device__ __forceinline__ float e4m3_sel(uint32_t w, int j) {
  return j == 0 ? e4m3_byte<0>(w) : j == 1 ? e4m3_byte<1>(w) : j == 2 ? e4m3_byte<2>(w) : e4m3_byte<3>(w);
}

// ---- scale step at the end of a cycle ------------------------------------
// c: cycle index inside the k-step when a k-step holds several cycles.
template <int FMT, int S>
__device__ __forceinline__ void flush(f32x4& acc, const f32x4& D, const f32x4& Db, const u32x4& sc, int c) {
  if constexpr (FMT == INT4 || FMT == INT5) {
    uint32_t w[4];
    if constexpr (S == 16) { w[0] = sc.x; w[1] = sc.z; w[2] = sc.y; w[3] = sc.w; }      // pos(i)
    else if constexpr (S == 1) {      // group c of the k-step, every A row: word pos(c)
      const uint32_t wc = c == 0 ? sc.x : c == 1 ? sc.z : c == 2 ? sc.y : sc.w;
      w[0] = w[1] = w[2] = w[3] = wc;
    }
    else if constexpr (S == 8) { w[0] = w[1] = sc.x; w[2] = w[3] = sc.y; }
    else if constexpr (S == 4) { w[0] = w[1] = w[2] = w[3] = sc.x; }
    else { w[0] = w[1] = w[2] = w[3] = (c == 0 ? sc.x : sc.y); }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float d = f16_lo(w[i]), m = f16_hi(w[i]);
      const float dq = D[i] - Db[i];                               // sum x q
      acc[i] = fmaf(m * CodeBias<FMT>::inv, Db[i], acc[i]);        // m sum x (m / c exact)
      acc[i] = fmaf(d, dq, acc[i]);
    }
  } else if constexpr (FMT == INT8) {
    float d[4];
    if constexpr (S == 16) { d[0] = f16_lo(sc.x); d[1] = f16_lo(sc.y); d[2] = f16_hi(sc.x); d[3] = f16_hi(sc.y); }
    else if constexpr (S == 1) {      // group c: fp16 at pos(c)
      const float dc = c == 0 ? f16_lo(sc.x) : c == 1 ? f16_lo(sc.y) : c == 2 ? f16_hi(sc.x) : f16_hi(sc.y);
      d[0] = d[1] = d[2] = d[3] = dc;
    }
    else if constexpr (S == 8) { d[0] = d[1] = f16_lo(sc.x); d[2] = d[3] = f16_lo(sc.y); }
    else if constexpr (S == 4) { d[0] = d[1] = d[2] = d[3] = f16_lo(sc.x); }
    else { d[0] = d[1] = d[2] = d[3] = (c == 0 ? f16_lo(sc.x) : f16_hi(sc.x)); }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(d[i], D[i], acc[i]);
  } else {
    float b[4];
    if constexpr (S == 16) {
      b[0] = e4m3_byte<0>(sc.x); b[1] = e4m3_byte<0>(sc.y); b[2] = e4m3_byte<1>(sc.x); b[3] = e4m3_byte<1>(sc.y);
    } else if constexpr (S == 8) {
      b[0] = b[1] = e4m3_byte<0>(sc.x); b[2] = b[3] = e4m3_byte<0>(sc.y);
    } else if constexpr (S == 4) {
      b[0] = b[1] = b[2] = b[3] = (c == 0 ? e4m3_byte<0>(sc.x) : e4m3_byte<2>(sc.x));
    } else {
      const float v = c == 0 ? e4m3_byte<0>(sc.x) : c == 1 ? e4m3_byte<1>(sc.x) : c == 2 ? e4m3_byte<2>(sc.x)
                                                                                         : e4m3_byte<3>(sc.x);
      b[0] = b[1] = b[2] = b[3] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(b[i], D[i], acc[i]);
  }
}

// Weight and scale descriptors of a k-loop: one buffer for all NT tiles (a
// plain descriptor), or one per tile (PerTile: tiles of different matrices,
// e.g. the same row tile of two experts).
template <int NT>
struct PerTile {
  __amdgpu_buffer_rsrc_t r[NT];
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rs_at(__amdgpu_buffer_rsrc_t r, int) { return r; }
template <int NT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rs_at(const PerTile<NT>& r, int t) { return r.r[t]; }

// Loads the packed weights of KPS k-steps starting at ks (wave-uniform) into
// st. K-steps at or past ks1 read as zeros (out-of-range offsets, no memory
// traffic).
// CYC: this buffer's first k-step starts a scale cycle of several k-steps;
// that cycle's scale words travel with the buffer, so they are in flight as
// long as the weights (a cycle's flush comes KSTEPS k-steps after its start).
template <int FMT, int NT, int S, int KPS, bool CYC, class WQ, class WS>
__device__ __forceinline__ void load_weights(Step<FMT, NT, KPS>& st, WQ wq, WS ws, const int (&tile)[NT], int KS,
                                             int ks, int ks1, uint32_t hi_offset) {
  const int lane = threadIdx.x & 63;
  constexpr int TB = FMT == INT8 ? 2048 : 1024;
#pragma unroll
  for (int i = 0; i < KPS; ++i) {
    const int k = ks + i;
    const bool ok = k < ks1;
    const uint32_t bad = ok ? 0u : 0x80000000u;
    const uint32_t lo = (uint32_t)lane * 16u | bad;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t tau = (uint32_t)tile[t] * (uint32_t)KS + (uint32_t)k;
      st.q[i][t] = ld128s_nt(rs_at(wq, t), lo, tau * TB);
      if constexpr (FMT == INT8) st.q2[i][t] = ld128s_nt(rs_at(wq, t), lo, tau * TB + 1024u);
      if constexpr (FMT == INT5)
        st.h[i][t] = ld32s_nt(rs_at(wq, t), (uint32_t)lane * 4u | bad, hi_offset + tau * 256u);
      if constexpr (Cyc<FMT, S>::KSTEPS == 1)
        st.sc[i][t] = load_scales<FMT, S>(rs_at(ws, t), tau, lane, ok ? 1 : 0);
      if constexpr (Cyc<FMT, S>::KSTEPS > 1 && CYC) {
        if (i == 0) st.cyc[t] = load_scales<FMT, S>(rs_at(ws, t), tau, lane, ks1 - k);
      }
    }
  }
}

// Activations of the 4 groups of k-step k (zeros past ks1 or past G).
// aload(g, adj): this lane's 8 activations of group g with the uniform offset
// adjustment adj added to its lane base. ckk: k-step position in its cycle.
template <int FMT, int S, class ALoad>
__device__ __forceinline__ void load_acts(bf16x8 (&A)[4], int k, int ks1, int G, int ckk, const ALoad& aload) {
  const bool ok = k < ks1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = k * 4 + j;
    const uint32_t adj = 0u - (uint32_t)slot_pos<FMT, S>(ckk, j) * kSlotStride + ((ok && g < G) ? 0u : 0x80000000u);
    A[j] = aload(g, adj);
  }
}

struct NoPrologue {
  __device__ void operator()() const {}
};

// KPS: k-steps per weight buffer; weights run one buffer ahead of the
// compute, activations AD k-steps ahead (1 everywhere: a deeper activation
// ring measured slower on MI355X, its registers cost more than the latency
// they hide). acts(A, k, pos) fetches the four A operands of k-step k,
// which sits at position pos of its loop trip (a compile-time constant at
// each call; its cycle position is pos % KSTEPS) — zeros past ks1 or past G;
// pre() runs once after the first weight loads are issued (EARLY: after
// the first two buffers', so a wave that waits in pre() has 2 * KPS k-steps
// of weights in flight meanwhile).
// kloop = kloop_start + kloop_run. A caller may run kloop_start itself,
// before its activation set-up: the wave's first weight loads then go out
// before any instruction that waits for kernel arguments still in flight.
// TB > 1 (one slot only): TB blocks of 16 tokens share every decoded weight
// operand; acts then fills A[TB][4] and acc[t * TB + b] holds block b of
// tile t.
template <int FMT, int NT, int S, int KPS, bool EARLY = false, class WQ, class WS>
__device__ __forceinline__ void kloop_start(Step<FMT, NT, KPS> (&buf)[2], WQ wq, WS ws, const int (&tile)[NT], int KS,
                                            int ks0, int ks1, uint32_t hi_offset) {
  using C = Cyc<FMT, S>;
  if (ks0 < ks1) {
    load_weights<FMT, NT, S, KPS, true>(buf[0], wq, ws, tile, KS, ks0, ks1, hi_offset);
    if constexpr (EARLY) {
      constexpr bool cyc1 = KPS % C::KSTEPS == 0;
      load_weights<FMT, NT, S, KPS, cyc1>(buf[1], wq, ws, tile, KS, ks0 + KPS, ks1, hi_offset);
    }
  }
  // nothing the scheduler could place in front of these loads
  __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int NT, int S, int KPS, int AD, int TB = 1, bool EARLY = false, bool PRIO = false, class WQ,
          class WS, class Acts, class Pre = NoPrologue>
__device__ __forceinline__ void kloop_run(Step<FMT, NT, KPS> (&buf)[2], WQ wq, WS ws, const int (&tile)[NT], int KS,
                                          int ks0, int ks1, uint32_t hi_offset, const Acts& acts,
                                          f32x4 (&acc)[NT * TB], const Pre& pre = Pre()) {
  static_assert(TB == 1 || S == 1, "token blocks need one slot");
  using C = Cyc<FMT, S>;
  constexpr int U = 2 * KPS;                     // k-steps per loop trip (a multiple of C::KSTEPS)
  constexpr int R = AD + 1;                      // activation ring
  static_assert(U % C::KSTEPS == 0, "cycle must divide the trip");
  // a buffer carries the scale words of at most one cycle, the one starting
  // at its first k-step (Step::cyc)
  static_assert(C::KSTEPS == 1 || (KPS <= C::KSTEPS && C::KSTEPS % KPS == 0),
                "a weight buffer may hold at most one scale-cycle start");
  static_assert(U % R == 0, "the activation ring must divide the trip");
  const bf16x8 bias_op = bf16x8_splat(FMT == INT5 ? kBias5Bits : kBias4Bits);   // int formats' code bias
  // HALVES: operand lanes 0-31 hold a group's columns 0-15 (block 0), lanes 32-63 columns 16-31 (block 1)
  const uint32_t lo_mask = (threadIdx.x & 32) ? 0u : 0xFFFFFFFFu;
  bf16x8 xa[R][TB][4];
  u32x4 csc[NT];                                 // scale words of the current cycle (KSTEPS > 1)
  f32x4 D[NT * TB];
  f32x4 Db[TB];
#pragma unroll
  for (int t = 0; t < NT; ++t) csc[t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < NT * TB; ++t) D[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < TB; ++b) Db[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ks0 >= ks1) return;
  auto fetch = [&](bf16x8 (&X)[TB][4], int k, int pos) {
    if constexpr (TB == 1) acts(X[0], k, pos);
    else acts(X, k, pos);
  };

  pre();
#pragma unroll
  for (int d = 0; d < AD; ++d) fetch(xa[d], ks0 + d, d);
  // PRIO: wave priority from the wave's own progress, 3 in the first
  // quarter of its range down to 0 in the last. The sequencer issues the
  // oldest ready wave first; where a unit holds more waves on some SIMDs than
  // on others, the younger waves there fall behind and finish last. Ranking
  // by progress instead lets a wave that lags catch up.
  const int pq = (ks1 - ks0) >> 2;
  const int pq1 = ks0 + pq, pq2 = ks0 + ((ks1 - ks0) >> 1), pq3 = ks1 - pq;
  for (int base = ks0; base < ks1; base += U) {
    if constexpr (PRIO) {
      if (base < pq1) __builtin_amdgcn_s_setprio(3);
      else if (base < pq2) __builtin_amdgcn_s_setprio(2);
      else if (base < pq3) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < KPS; ++i) {
        const int kk = b * KPS + i;                // k-step index in the trip
        const int ks = base + kk;
        const int ckk = kk % C::KSTEPS;            // k-step position inside its cycle
        if (i == 0) {                              // next weight buffer (and its cycle's scales)
          constexpr bool cyc1 = KPS % C::KSTEPS == 0;        // buffer base + KPS starts a cycle
          constexpr bool cyc2 = (2 * KPS) % C::KSTEPS == 0;  // buffer base + 2 KPS does
          if (b == 0) {
            if (!EARLY || base != ks0) load_weights<FMT, NT, S, KPS, cyc1>(buf[1], wq, ws, tile, KS, base + KPS, ks1, hi_offset);
          }
          else load_weights<FMT, NT, S, KPS, cyc2>(buf[0], wq, ws, tile, KS, base + 2 * KPS, ks1, hi_offset);
        }
        fetch(xa[(kk + AD) % R], ks + AD, (kk + AD) % U);
        if constexpr (C::KSTEPS > 1) {
          if (ckk == 0) {                          // cycle start: its scale words came with this buffer
#pragma unroll
            for (int t = 0; t < NT; ++t) csc[t] = buf[b].cyc[t];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        const Step<FMT, NT, KPS>& cur = buf[b];
        bf16x8 B5[NT][4];
        if constexpr (FMT == INT5) {
#pragma unroll
          for (int t = 0; t < NT; ++t) dec_int5_step(cur.q[i][t], cur.h[i][t], B5[t]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (C::HALVES) {
            bf16x8 Ah[TB][2];                      // block 0 / block 1 activations, the other block's lanes zero
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              const u32x4 v = __builtin_bit_cast(u32x4, xa[kk % R][tb][j]);
              const u32x4 v0 = {v.x & lo_mask, v.y & lo_mask, v.z & lo_mask, v.w & lo_mask};
              const u32x4 v1 = {v.x & ~lo_mask, v.y & ~lo_mask, v.z & ~lo_mask, v.w & ~lo_mask};
              Ah[tb][0] = __builtin_bit_cast(bf16x8, v0);
              Ah[tb][1] = __builtin_bit_cast(bf16x8, v1);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const u32x4 q = cur.q[i][t];
              const bf16x8 B = dec_nvfp4(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w);
              const u32x4 sc = cur.sc[i][t];
              const float b0 = e4m3_sel(sc.x, j), b1 = e4m3_sel(sc.y, j);
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) {
                const f32x4 D0 = mfma(Ah[tb][0], B, f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 D1 = mfma(Ah[tb][1], B, f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4& A = acc[t * TB + tb];
#pragma unroll
                for (int e = 0; e < 4; ++e) A[e] = fmaf(b1, D1[e], fmaf(b0, D0[e], A[e]));
              }
            }
          } else {
            const int gpos = 4 * ckk + j;            // group position in the cycle
            const bool first = (gpos % C::GROUPS) == 0;
            const bool last = ((gpos + 1) % C::GROUPS) == 0;
            const int cidx = gpos / C::GROUPS;       // cycle index inside the k-step
            if constexpr (FMT == INT4 || FMT == INT5) {
#pragma unroll
              for (int tb = 0; tb < TB; ++tb)
                Db[tb] = mfma(xa[kk % R][tb][j], bias_op, first ? f32x4{0.f, 0.f, 0.f, 0.f} : Db[tb]);
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              bf16x8 B;
              const u32x4 q = cur.q[i][t];
              if constexpr (FMT == INT4) {
                B = dec_int4(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w);
              } else if constexpr (FMT == INT5) {
                B = B5[t][j];
              } else if constexpr (FMT == INT8) {
                const u32x4 qq = j < 2 ? q : cur.q2[i][t];
                B = (j & 1) ? dec_int8(qq.z, qq.w) : dec_int8(qq.x, qq.y);
              } else {
                B = dec_nvfp4(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w);
              }
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) {
                f32x4& Dt = D[t * TB + tb];
                Dt = mfma(xa[kk % R][tb][j], B, first ? f32x4{0.f, 0.f, 0.f, 0.f} : Dt);
                if (last) {
                  if constexpr (C::KSTEPS > 1) flush<FMT, S>(acc[t * TB + tb], Dt, Db[tb], csc[t], cidx);
                  else flush<FMT, S>(acc[t * TB + tb], Dt, Db[tb], cur.sc[i][t], cidx);
                }
              }
            }
          }
        }
      }
    }
  }
  if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

template <int FMT, int NT, int S, int KPS, int AD, int TB = 1, bool EARLY = false, class Acts, class Pre = NoPrologue>
__device__ __forceinline__ void kloop(__amdgpu_buffer_rsrc_t wq, __amdgpu_buffer_rsrc_t ws, const int (&tile)[NT],
                                      int KS, int ks0, int ks1, uint32_t hi_offset, const Acts& acts,
                                      f32x4 (&acc)[NT * TB], const Pre& pre = Pre()) {
  Step<FMT, NT, KPS> buf[2];
  kloop_start<FMT, NT, S, KPS, EARLY>(buf, wq, ws, tile, KS, ks0, ks1, hi_offset);
  kloop_run<FMT, NT, S, KPS, AD, TB, EARLY>(buf, wq, ws, tile, KS, ks0, ks1, hi_offset, acts, acc, pre);
}

}  // namespace qg
