// Mixture-of-experts path (qgemv_moe, qgemv_moe_index, qgemv_moe_workspace_bytes).
//
// What it computes (Decapybara page, CUDA kernel list: a top-8 softmax MoE
// router; memra page: a 35B-A3B MoE served from one card; NInfer article,
// section 2: SwiGLU fused into the matmul): every token t runs only the
// experts it selected, y[t] = r[t] + sum_j p[t][j] * down_e(SwiGLU(gate_up_e(x[t]))).
//
// Three launches on one stream, no host synchronisation:
//   1. gate/up + SwiGLU: grid (row tiles, active-expert slot). Each
//      workgroup first routes in LDS (one wave, exact integer work on the
//      <= 64 selected ids): the a-th smallest selected expert and the (token,
//      slot) pairs routed to it in (token, slot) order; a slot past the number
//      of selected experts exits at once. It then gathers the rows of x routed
//      to its expert (8 per MFMA pass) and writes h [pair][I].
//   2. down: same grid shape over H and the same routing. h leaves step 1 as a pair of bf16 planes
//      hi = bf16(h), lo = bf16(h - hi) (h = hi + lo + O(2^-16 |h|), the same
//      bytes as fp32), so the A operand holds 4 pairs x {hi, lo} x 2 slots;
//      writes o [pair][H] in fp32.
// The routing index itself (counts, offsets, pairs in (expert, token, slot)
// order, active experts, error flag) is qgemv_moe_index, one workgroup.
//   3. combine: y[t] = r[t] + sum_j p[t][j] o[t*k + j] in increasing j order;
//      no atomics, so results are bitwise reproducible (RustingStrata page,
//      known issues: run-to-run reordering changes results).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "device.hpp"
#include "kloop.hpp"
#include "layout.hpp"
#include "qgemv.h"
#include "route.hpp"

namespace qg {

// ---- routing (exact integer work on the N * top_k <= 64 selected ids) -----

// Largest expert count qgemv_moe accepts: the routing bitmap lives in LDS.
constexpr int kMaxExperts = 16384;

// Active slot a -> expert, in LDS, for one whole wave: s_route[0] = the a-th
// smallest selected expert id (-1 if fewer than a + 1 experts are selected),
// s_route[1] = the number of pairs routed to it, s_route[2..] = those flat
// entries t * top_k + j, ascending. A bitmap of selected experts (OR is
// order-independent) is scanned with one prefix sum over the lanes' chunks.
__device__ __forceinline__ void route_slot(int id, int NK, int E, int a, uint32_t* s_bits, int* s_route) {
  const int lane = threadIdx.x & 63;
  const int W = (E + 31) >> 5, c = (W + 63) >> 6;   // bitmap words, words per lane
  for (int i = 0; i < c; ++i) {
    const int w = lane * c + i;
    if (w < W) s_bits[w] = 0u;
  }
  // id: the lane's entry (lane < NK; anything elsewhere)
  const int v = (lane < NK && id >= 0 && id < E) ? id : -1;
  // one wave: its LDS operations complete in issue order (clears, ORs, reads)
  __builtin_amdgcn_wave_barrier();
  if (v >= 0) atomicOr(s_bits + (v >> 5), 1u << (v & 31));
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
  for (int i = 0; i < c; ++i) {
    const int w = lane * c + i;
    if (w < W) cnt += __builtin_popcount(s_bits[w]);
  }
  int incl = cnt;                 // inclusive prefix sum over lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  const int n_active = __shfl(incl, 63);
  int e = -1;
  if (a < n_active && incl - cnt <= a && a < incl) {
    int rem = a - (incl - cnt);
    for (int i = 0; i < c && e < 0; ++i) {
      const int w = lane * c + i;
      uint32_t bits = w < W ? s_bits[w] : 0u;
      const int pc = __builtin_popcount(bits);
      if (rem < pc) {
        for (int r = 0; r < rem; ++r) bits &= bits - 1u;   // drop the lowest rem set bits
        e = 32 * w + __builtin_ctz(bits);
      } else {
        rem -= pc;
      }
    }
  }
  const uint64_t owner = __ballot(e >= 0);
  e = owner ? __shfl(e, __builtin_ctzll(owner)) : -1;
  const uint64_t mine = __ballot(e >= 0 && v == e);
  if (e >= 0 && v == e) s_route[2 + __builtin_popcountll(mine & ((1ull << lane) - 1ull))] = lane;
  if (lane == 0) {
    s_route[0] = e;
    s_route[1] = __builtin_popcountll(mine);
  }
}

// Per-slot routing of every active expert at once (one wave), as the
// single-launch MoE runs it: slot a = the a-th smallest selected expert,
// slot_e[a], its entries' offset slot_off[a] and count slot_cnt[a], and
// pairs[slot_off[a] ..) those flat entries t * top_k + j in (t, j) order.
// Lane i holds entry i (i < NK); every comparison with another entry reads
// that entry's id from its lane (v_readlane, a scalar result), so the work
// is a few register operations per entry with no memory round trips.
// Returns the number of active experts (every lane).
__device__ __forceinline__ int index_lanes(const int32_t* ids, int NK, int E, int* pairs, int* slot_e, int* slot_off,
                                           int* slot_cnt) {
  const int lane = threadIdx.x & 63;
  int v = -2;                    // -1: outside [0, E); -2: past NK
  if (lane < NK) {
    const int id = ids[lane];
    v = (id >= 0 && id < E) ? id : -1;
  }
  bool first = v >= 0;           // first occurrence of its expert among the entries
  int below = 0, same_before = 0, same = 0;
  for (int j = 0; j < NK; ++j) {
    const int u = __builtin_amdgcn_readlane(v, j);
    below += u >= 0 && u < v;
    same += u == v;
    if (j < lane && u == v) {
      ++same_before;
      first = false;
    }
  }
  const uint64_t act = __ballot(first);
  int rank = 0;                  // active experts with a smaller id
  for (uint64_t m = act; m; m &= m - 1) rank += __builtin_amdgcn_readlane(v, (int)__builtin_ctzll(m)) < v;
  if (v >= 0) {
    pairs[below + same_before] = lane;
    if (first) {
      slot_e[rank] = v;
      slot_off[rank] = below;
      slot_cnt[rank] = same;
    }
  }
  return __builtin_popcountll(act);
}

// Routing index dump (qgemv_moe_index_by): one workgroup of 256 threads.
// ROUTINE 0 runs route_slot once per slot, exactly as every expert
// workgroup of qgemv_moe does; ROUTINE 1 runs index_lanes, as every
// workgroup of the single-launch qgemv_moe_fused does. Both leave per-slot
// (expert, offset, count) and the pairs in LDS, from which the full index is
// written: counts and offsets for every expert, pairs, active list, and
// meta = {active experts, 1 if some entry was outside [0, E)}.
template <int ROUTINE>
__global__ __launch_bounds__(256) void k_moe_index(const int32_t* ids, int NK, int E, int32_t* counts,
                                                   int32_t* offsets, int32_t* pairs, int32_t* active,
                                                   int32_t* meta) {
  __shared__ uint32_t s_bits[kMaxExperts / 32];
  __shared__ int s_route[2 + 64];
  __shared__ int s_pairs[64];
  __shared__ int s_slot_e[64], s_slot_off[64], s_slot_cnt[64];
  __shared__ int s_meta[2];               // active experts, routed entries
  const int tid = threadIdx.x;
  if (tid < 64) {
    if constexpr (ROUTINE == 0) {
      int a = 0, off = 0;
      const int id = tid < NK ? ids[tid] : 0;
      for (; a < min(E, NK); ++a) {
        route_slot(id, NK, E, a, s_bits, s_route);
        __builtin_amdgcn_wave_barrier();
        const int e = s_route[0], cnt = s_route[1];
        if (e < 0) break;                 // uniform: fewer selected experts than slots
        if (tid < cnt) s_pairs[off + tid] = s_route[2 + tid];
        if (tid == 0) {
          s_slot_e[a] = e;
          s_slot_off[a] = off;
          s_slot_cnt[a] = cnt;
        }
        off += cnt;
        __builtin_amdgcn_wave_barrier();  // s_route is rewritten by the next slot
      }
      if (tid == 0) {
        s_meta[0] = a;
        s_meta[1] = off;
      }
    } else {
      const int n = index_lanes(ids, NK, E, s_pairs, s_slot_e, s_slot_off, s_slot_cnt);
      __builtin_amdgcn_wave_barrier();
      if (tid == 0) {
        int tot = 0;
        for (int a = 0; a < n; ++a) tot += s_slot_cnt[a];
        s_meta[0] = n;
        s_meta[1] = tot;
      }
    }
  }
  __syncthreads();
  const int n_active = s_meta[0], routed = s_meta[1];
  for (int p = tid; p < NK; p += blockDim.x) pairs[p] = p < routed ? s_pairs[p] : -1;
  for (int e = tid; e < E; e += blockDim.x) {
    int c = 0, below = 0;
    for (int a = 0; a < n_active; ++a) {
      c += s_slot_e[a] == e ? s_slot_cnt[a] : 0;
      below += s_slot_e[a] < e ? s_slot_cnt[a] : 0;
    }
    counts[e] = c;
    offsets[e] = below;
    active[e] = e < n_active ? s_slot_e[e] : -1;
  }
  if (tid == 0) {
    offsets[E] = routed;
    meta[0] = n_active;
    meta[1] = routed < NK ? 1 : 0;
  }
}

struct MoeArgs {
  const uint8_t* wq;
  const uint8_t* ws;
  uint64_t wq_stride, ws_stride;   // bytes between experts
  uint32_t wq_bytes, ws_bytes;     // one expert's packed sizes
  uint32_t hi_offset, st_offset;
  const void* in;                  // gate/up: x bf16 [N][K]; down: h as bf16 hi and lo planes [2][NK][K]
  uint32_t in_bytes;
  float* out;                      // gate/up: h planes (bf16) [2][NK][Mout]; down: o fp32 [NK][Mout]
  uint32_t out_bytes;
  const int32_t* ids;              // [N][top_k] selected experts
  int E, top_k, NK;
  int Mout, K, KS, G;
  int out_tiles, up_tile0;
  int ks_per_wave;
};

// hi/lo bf16 split of an fp32 value: hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = (__bf16)v;
  lo = (__bf16)(v - (float)hi);
}

// Buffer accesses at device scope (cache policy sc1): they bypass the
// per-XCD caches that are not coherent with each other, so data one
// workgroup writes this way is seen by a workgroup on another XCD once the
// writer's stores have completed (s_waitcnt) before it bumps a counter.
constexpr int kDeviceScope = 16;
__device__ __forceinline__ u32x4 ld128s_dev(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kDeviceScope);
}
__device__ __forceinline__ float ld_f32_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kDeviceScope));
}

struct NoWait {
  __device__ void operator()() const {}
};

// One work item of the expert GEMVs: output row block rb of expert e for
// the cnt routed entries pairs[0..cnt) (flat t * top_k + j, ascending).
// DOWN = false: gate/up + SwiGLU (NT = 2*TO tiles: gate then up)
// DOWN = true:  down projection (NT = TO tiles)
// COH: the item runs inside the single-launch MoE kernel, where another
// workgroup consumes its output: outputs are stored at device scope, and the
// down projection reads h at device scope after wait() (run by every wave
// once its first weight loads are in flight) has seen h complete.
// red: LDS of W * NT * 32 * 4 floats. Ends with a workgroup barrier.
template <int FMT, int NT, bool DOWN, bool COH, class Wait = NoWait>
__device__ __forceinline__ void moe_item(const MoeArgs& a, int e, int cnt, const int* pairs, int rb, float* red,
                                         const Wait& wait = Wait()) {
  constexpr int TO = DOWN ? NT : NT / 2;
  constexpr int ROWS = DOWN ? 4 : 8;   // routed rows per MFMA pass
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane & 15, s = lane >> 4;

  const __amdgpu_buffer_rsrc_t wq = make_rsrc(a.wq + (uint64_t)e * a.wq_stride, a.wq_bytes);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.ws + (uint64_t)e * a.ws_stride, a.ws_bytes);
  const __amdgpu_buffer_rsrc_t inr = make_rsrc(a.in, a.in_bytes);
  const __amdgpu_buffer_rsrc_t outr = make_rsrc(a.out, a.out_bytes);

  int tile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int ot = rb * TO + (t % TO);
    ot = ot < a.out_tiles ? ot : a.out_tiles - 1;
    tile[t] = (!DOWN && t >= TO) ? a.up_tile0 + ot : ot;
  }
  const int ks0 = wave * a.ks_per_wave;
  const int ks1 = min(a.KS, ks0 + a.ks_per_wave);
  float st = 1.0f;
  if constexpr (FMT == NVFP4) st = __builtin_bit_cast(float, ld32(ws, a.st_offset));

  for (int c0 = 0; c0 < cnt; c0 += ROWS) {
    const int nrows = min(ROWS, cnt - c0);
    // this lane's routed row (A row r): gate/up token = r & 7; down pair = r & 3
    const int ar = DOWN ? (r & 3) : (r & 7);
    const bool row_ok = ar < nrows;
    const int pflat = row_ok ? pairs[c0 + ar] : 0;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t slot_term = lane_slot_term<FMT, 2>(lane);
    if constexpr (!DOWN) {
      const uint32_t base = (row_ok ? (uint32_t)((pflat / a.top_k) * a.K + 8 * s) * 2u : kAbsentRow) + slot_term;
      auto aload = [&](int g, uint32_t adj) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, ld128s(inr, base + adj, (uint32_t)g * 64u));
      };
      auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
        load_acts<FMT, 2>(A, k, ks1, a.G, pos % Cyc<FMT, 2>::KSTEPS, aload);
      };
      kloop<FMT, NT, 2, 2, 1>(wq, ws, tile, a.KS, ks0, ks1, a.hi_offset, acts, acc);
    } else {
      // A rows 8*slot + 4*part + pair: part 0 reads the hi plane of h, part 1 the lo plane
      const int part = (r >> 2) & 1;
      const uint32_t base = (row_ok ? (uint32_t)((part * a.NK + pflat) * a.K + 8 * s) * 2u : kAbsentRow) + slot_term;
      auto aload = [&](int g, uint32_t adj) -> bf16x8 {
        if constexpr (COH) return __builtin_bit_cast(bf16x8, ld128s_dev(inr, base + adj, (uint32_t)g * 64u));
        return __builtin_bit_cast(bf16x8, ld128s(inr, base + adj, (uint32_t)g * 64u));
      };
      auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
        load_acts<FMT, 2>(A, k, ks1, a.G, pos % Cyc<FMT, 2>::KSTEPS, aload);
      };
      // the wait runs once per item, before the first pass reads h
      if (c0 == 0) kloop<FMT, NT, 2, 2, 1>(wq, ws, tile, a.KS, ks0, ks1, a.hi_offset, acts, acc, wait);
      else kloop<FMT, NT, 2, 2, 1>(wq, ws, tile, a.KS, ks0, ks1, a.hi_offset, acts, acc);
    }
    // reduce: slots (lane ^ 32); for DOWN also hi/lo parts (lane ^ 16)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[t][i] += __shfl_xor(acc[t][i], 32);
        if constexpr (DOWN) acc[t][i] += __shfl_xor(acc[t][i], 16);
      }
    }
    constexpr int LANES = DOWN ? 16 : 32;
    if (lane < LANES) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float* p = red + (((size_t)wave * NT + t) * 32 + lane) * 4;
        p[0] = acc[t][0];
        p[1] = acc[t][1];
        p[2] = acc[t][2];
        p[3] = acc[t][3];
      }
    }
    __syncthreads();
    const int n_out = TO * 16 * ROWS;
    for (int o = threadIdx.x; o < n_out; o += blockDim.x) {
      const int to = o / (16 * ROWS), rem = o % (16 * ROWS);
      const int rr = rem / 16, row = rem % 16;
      const int ot = rb * TO + to;
      const int col = ot * 16 + row;
      if (rr >= nrows || ot >= a.out_tiles || col >= a.Mout) continue;
      const int l = DOWN ? row : row + 16 * (rr >> 2), i = DOWN ? rr : (rr & 3);
      float v = 0.f;
      for (int w = 0; w < W; ++w) v += red[(((size_t)w * NT + to) * 32 + l) * 4 + i];
      v *= st;
      const int pf = pairs[c0 + rr];
      if constexpr (DOWN) {
        if constexpr (COH) {
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), outr,
                                                (uint32_t)(pf * a.Mout + col) * 4u, 0, kDeviceScope);
        } else {
          a.out[(size_t)pf * a.Mout + col] = v;
        }
      } else {
        float u = 0.f;
        for (int w = 0; w < W; ++w) u += red[(((size_t)w * NT + TO + to) * 32 + l) * 4 + i];
        u *= st;
        const float hv = v / (1.0f + expf(-v)) * u;
        __bf16 hi, lo;
        split_bf16(hv, hi, lo);
        if constexpr (COH) {
          const uint32_t o0 = (uint32_t)(pf * a.Mout + col) * 2u, o1 = (uint32_t)((a.NK + pf) * a.Mout + col) * 2u;
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hi), outr, o0, 0, kDeviceScope);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, lo), outr, o1, 0, kDeviceScope);
        } else {
          __bf16* hs = (__bf16*)a.out;             // hi plane [NK][I], then lo plane
          hs[(size_t)pf * a.Mout + col] = hi;
          hs[((size_t)a.NK + pf) * a.Mout + col] = lo;
        }
      }
    }
    __syncthreads();
  }
}

// Grid (row blocks, active-expert slot): routes in LDS, then one item.
// ids, NK, E: copies of a's fields, leading scalar arguments so that they are
// preloaded into SGPRs at wave launch and the ids load goes out at once.
template <int FMT, int NT, bool DOWN>
__global__ __launch_bounds__(512) void k_moe_gemv(const int32_t* ids, int NK, int E, MoeArgs a) {
  extern __shared__ float red[];  // [W][NT][32][4]
  __shared__ uint32_t s_bits[kMaxExperts / 32];
  __shared__ int s_route[2 + 64];
  const int lane = threadIdx.x & 63;
  const int id = (threadIdx.x < 64 && lane < NK) ? ids[lane] : 0;
  // the expert GEMV's arguments in one batch while the ids load is in flight
  asm volatile("" ::"s"(a.wq), "s"(a.ws), "s"(a.wq_stride), "s"(a.ws_stride), "s"(a.wq_bytes), "s"(a.ws_bytes),
               "s"(a.hi_offset), "s"(a.st_offset), "s"(a.in), "s"(a.in_bytes), "s"(a.KS), "s"(a.ks_per_wave),
               "s"(a.out_tiles), "s"(a.up_tile0), "s"(a.K), "s"(a.G));
  if (threadIdx.x < 64) route_slot(id, NK, E, blockIdx.y, s_bits, s_route);
  __syncthreads();
  // values read from LDS are the same in every lane: readfirstlane makes that
  // visible to the compiler (scalar branches, buffer descriptors in SGPRs)
  const int e = uniform(s_route[0]);
  if (e < 0) return;                   // fewer selected experts than slots
  moe_item<FMT, NT, DOWN, false>(a, e, uniform(s_route[1]), s_route + 2, blockIdx.x, red);
}

__global__ __launch_bounds__(256) void k_moe_combine(const float* o, const int32_t* ids, const float* gates,
                                                     const float* res, float* y, int N, int H, int top_k,
                                                     int E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * H) return;
  const int t = (int)(i / H), col = (int)(i % H);
  // every load first (independent), then the fixed-order sum
  float ov[8], pv[8];
  int ev[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < top_k) {
      ev[j] = ids[t * top_k + j];
      pv[j] = gates[t * top_k + j];
      ov[j] = o[(size_t)(t * top_k + j) * H + col];
    }
  }
  float v = res ? res[i] : 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < top_k && ev[j] >= 0 && ev[j] < E) v = fmaf(pv[j], ov[j], v);
  y[i] = v;
}

// qgemv_moe_route: one wave per token, 4 tokens per workgroup.
__global__ __launch_bounds__(256) void k_moe_route(const float* logits, int N, int E, int top_k, int32_t* ids,
                                                   float* gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;                 // uniform per wave
  const int lane = threadIdx.x & 63;
  int id;
  float g;
  route_token_any(logits + (size_t)t * E, E, top_k, &id, &g);
  if (lane < top_k) {
    ids[t * top_k + lane] = id;
    gates[t * top_k + lane] = g;
  }
}

// ---- single-launch MoE FFN (few routed rows) ---------------------------------
// One workgroup of FW waves per work item, launched in item order: first one
// item per (slot, gate/up row block), then one per 16-column block of the
// output y.
//   gate/up item: writes its rows of h at device scope, waits until those
//     stores have completed, and raises its own flag (slot, row block) to
//     this call's epoch: one store, no read-modify-write on the way.
//   output item: wave w computes o = h . W_dn[e] for slots w and w + FW
//     over the whole K. Both experts' weight loads are issued first; then it polls the
//     flags of every row block of its slot (one load per lane, bounded) until
//     all hold the epoch, and reads h at device scope. The o values meet in
//     LDS and the workgroup sums y = r + sum_j p_j o_j in fixed j order.
// Epochs: the host numbers the calls of the process 1, 2, ... (64-bit, so
// they never repeat), so a flag left by an earlier call on the same
// workspace never matches and nothing has to be cleared after use.
// Deadlock-free without co-residency: workgroups are dispatched in increasing
// order on every XCD, gate/up workgroups precede every output workgroup and
// never wait, so a waiting wave only waits for workgroups already running or
// done. A time-out sets the sticky error word and lets the kernel finish.
struct MoeFusedArgs {
  MoeArgs g[2];            // [0] gate/up items (grid row 0), [1] output items (grid row 1)
  const float* logits;     // [N][E]
  const float* res;        // [N][H] or null
  float* y;                // [N][H]
  int32_t* ids_out;        // [N][top_k] or null
  float* gates_out;        // [N][top_k] or null
  uint32_t* ctr;           // workspace: sticky error word, then the item flags
  uint64_t epoch;          // this call's number (> 0)
  int N, H, E, top_k, NK, slots;
  int nA, nB;              // gate/up row blocks per slot; 16-column output blocks
};
constexpr int kFusedMaxRows = 8;            // N * top_k handled by the single launch
// workspace words: [3] sticky error; 64-bit item flags [slot][row block] from byte 256
constexpr int kCtrError = 3;
constexpr int kFlagByte = 256;
constexpr uint32_t kSpinLimit = 1u << 20;   // polls before a wait gives up

// Waves per workgroup. Eight (one output expert per wave at eight active
// experts) measured 12% slower on the 128-expert top-8 workload at N = 1:
// the extra output waves' weight loads queue in front of the gate/up items'.
constexpr int kFusedWaves = 4;

// Hand-offs between workgroups use agent-scope atomics with relaxed order:
// h is written and read with device-scope (sc1) buffer accesses, which
// bypass the per-XCD L2s and complete at the coherence point. A gate/up
// item's threads wait for their h stores to complete (s_waitcnt) and meet at
// a barrier before thread 0 stores the item's flag, so the flag cannot run
// ahead of the data; an output wave issues its h loads only after its poll
// has returned every flag of its slot (a value-dependent branch; the signal
// fence keeps the compiler from hoisting the loads). Release/acquire at
// agent scope would add an L2 writeback / invalidate per hand-off: on the
// dense split remainder that measured 2x slower.
__device__ __forceinline__ uint64_t flag_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// o of one expert for one 16-row tile of the down projection, computed by one
// wave over the whole K: o_lds[pair][row] for the expert's cnt pairs. pre:
// the expert's first two weight buffers, already issued by
// kloop_start<FMT, 1, 2, 3, true> on this expert's descriptors and tile rt
// (the first pass of four routed rows continues from them). h is read at
// device scope after wait() has seen it complete.
template <int FMT, class Wait>
__device__ __forceinline__ void down_tile_wave(const MoeArgs& a, int e, int cnt, const int* pairs, int rt,
                                               float* o_lds, const Wait& wait, Step<FMT, 1, 3> (&pre)[2]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, s = lane >> 4;
  const __amdgpu_buffer_rsrc_t wq = make_rsrc(a.wq + (uint64_t)e * a.wq_stride, a.wq_bytes);
  const __amdgpu_buffer_rsrc_t ws = make_rsrc(a.ws + (uint64_t)e * a.ws_stride, a.ws_bytes);
  const __amdgpu_buffer_rsrc_t inr = make_rsrc(a.in, a.in_bytes);
  const int tile[1] = {rt};
  float st = 1.0f;
  if constexpr (FMT == NVFP4) st = __builtin_bit_cast(float, ld32(ws, a.st_offset));
  const uint32_t slot_term = lane_slot_term<FMT, 2>(lane);
  for (int c0 = 0; c0 < cnt; c0 += 4) {
    const int nrows = min(4, cnt - c0);
    const int ar = r & 3;
    const bool row_ok = ar < nrows;
    const int pflat = row_ok ? pairs[c0 + ar] : 0;
    const int part = (r >> 2) & 1;   // A rows 8*slot + 4*part + pair: hi / lo plane of h
    const uint32_t base = (row_ok ? (uint32_t)((part * a.NK + pflat) * a.K + 8 * s) * 2u : kAbsentRow) + slot_term;
    auto aload = [&](int g, uint32_t adj) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, ld128s_dev(inr, base + adj, (uint32_t)g * 64u));
    };
    auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
      load_acts<FMT, 2>(A, k, a.KS, a.G, pos % Cyc<FMT, 2>::KSTEPS, aload);
    };
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    if (c0 == 0) kloop_run<FMT, 1, 2, 3, 1, 1, true>(pre, wq, ws, tile, a.KS, 0, a.KS, a.hi_offset, acts, acc, wait);
    else kloop<FMT, 1, 2, 3, 1>(wq, ws, tile, a.KS, 0, a.KS, a.hi_offset, acts, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][i] += __shfl_xor(acc[0][i], 32);   // slots
      acc[0][i] += __shfl_xor(acc[0][i], 16);   // hi + lo parts
    }
    if (lane < 16 && rt * 16 + lane < a.Mout) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nrows) o_lds[pairs[c0 + i] * 16 + lane] = acc[0][i] * st;
    }
  }
}

// o of two experts for one 16-row tile of the down projection, in one k-loop
// by one wave: the experts' weight tiles are the loop's two tiles (one
// descriptor each) and their routed pairs share the A operand (pairs 0..n0-1
// of the first expert, then n1 of the second; n0 + n1 <= 4). Tile t's dot
// products with the other expert's rows are computed and dropped; in return
// the two experts' MFMA and decode chains interleave instead of running one
// after the other. pre: both tiles' first two weight buffers, already issued
// by kloop_start<FMT, 2, 2, 3, true>. h is read at device scope: the caller
// has seen both slots complete.
template <int FMT>
__device__ __forceinline__ void down_pair_wave(const MoeArgs& a, PerTile<2> wq, PerTile<2> ws, int n0, int n1,
                                               const int* p0, const int* p1, int rt, float* o_lds,
                                               Step<FMT, 2, 3> (&pre)[2]) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, s = lane >> 4;
  const __amdgpu_buffer_rsrc_t inr = make_rsrc(a.in, a.in_bytes);
  const int tile[2] = {rt, rt};
  float st0 = 1.0f, st1 = 1.0f;
  if constexpr (FMT == NVFP4) {
    st0 = __builtin_bit_cast(float, ld32(ws.r[0], a.st_offset));
    st1 = __builtin_bit_cast(float, ld32(ws.r[1], a.st_offset));
  }
  const int ar = r & 3;
  const bool row_ok = ar < n0 + n1;
  const int pflat = ar < n0 ? p0[ar] : (row_ok ? p1[ar - n0] : 0);
  const int part = (r >> 2) & 1;   // A rows 8*slot + 4*part + pair: hi / lo plane of h
  const uint32_t base = (row_ok ? (uint32_t)((part * a.NK + pflat) * a.K + 8 * s) * 2u : kAbsentRow) +
                        lane_slot_term<FMT, 2>(lane);
  auto aload = [&](int g, uint32_t adj) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, ld128s_dev(inr, base + adj, (uint32_t)g * 64u));
  };
  auto acts = [&](bf16x8 (&A)[4], int k, int pos) {
    load_acts<FMT, 2>(A, k, a.KS, a.G, pos % Cyc<FMT, 2>::KSTEPS, aload);
  };
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  kloop_run<FMT, 2, 2, 3, 1, 1, true>(pre, wq, ws, tile, a.KS, 0, a.KS, a.hi_offset, acts, acc);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[t][i] += __shfl_xor(acc[t][i], 32);   // slots
      acc[t][i] += __shfl_xor(acc[t][i], 16);   // hi + lo parts
    }
  }
  if (lane < 16 && rt * 16 + lane < a.Mout) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < n0) o_lds[p0[i] * 16 + lane] = acc[0][i] * st0;
      else if (i < n0 + n1) o_lds[p1[i - n0] * 16 + lane] = acc[1][i] * st1;
    }
  }
}

// logits, E, top_k, N: copies of f's fields, leading scalar arguments
// preloaded into SGPRs at wave launch, so each wave's first logits load goes
// out at once.
template <int FMT>
__global__ __launch_bounds__(64 * kFusedWaves) void k_moe_fused(const float* logits, int E, int top_k, int N,
                                                                MoeFusedArgs f) {
  constexpr int FW = kFusedWaves;
  extern __shared__ __attribute__((aligned(16))) float red[];   // [FW][2][32][4] (gate/up), then o [8][16]
  __shared__ int32_t s_ids[64];
  __shared__ float s_gates[64];
  __shared__ int s_pairs[64];
  __shared__ int s_slot_e[64], s_slot_off[64], s_slot_cnt[64];
  __shared__ int s_meta[1];               // active experts
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int row = blockIdx.y;              // 0: gate/up items, 1: output items
  const int tk = blockIdx.x;
  // This workgroup's expert GEMV arguments, fetched with everything else
  // before the router runs: the grid row selects them without a load, and
  // the empty asm takes them as scalar-register inputs, so their loads go
  // out in the kernel's first batch instead of one dependent round trip to
  // the argument block at a time further down.
  // the wave's first token: its keys' logits load goes out before the batch
  // below (E <= 128, the register-cached router)
  float lv0[2] = {0.0f, 0.0f};
  if (E <= 128 && wave < N) route_logits<2>(logits + (size_t)wave * E, E, lv0);
  const MoeArgs m = f.g[row];
  asm volatile("" ::"s"(m.wq), "s"(m.ws), "s"(m.wq_stride), "s"(m.ws_stride), "s"(m.wq_bytes), "s"(m.ws_bytes),
               "s"(m.hi_offset), "s"(m.st_offset), "s"(m.in), "s"(m.in_bytes), "s"(m.out), "s"(m.out_bytes),
               "s"(m.NK), "s"(m.Mout), "s"(m.K), "s"(m.KS), "s"(m.G), "s"(m.out_tiles), "s"(m.up_tile0),
               "s"(m.ks_per_wave), "s"(f.nA), "s"(f.NK), "s"(f.slots), "s"(f.nB)
               : "memory");
  if (tk >= (row == 0 ? f.slots * f.nA : f.nB)) return;   // the shorter row's spare workgroups

  // router: every workgroup routes every token itself (no launch, no wait),
  // one wave per token
  for (int t = wave; t < N; t += FW) {
    int id;
    float g;
    if (E <= 128 && t == wave) {
      uint64_t key0[2];
      route_keys<2>(lv0, E, key0);
      route_select<2>(key0, nullptr, E, top_k, &id, &g);
    }
    else route_token_any(logits + (size_t)t * E, E, top_k, &id, &g);
    if (lane < top_k) {
      s_ids[t * top_k + lane] = id;
      s_gates[t * top_k + lane] = g;
    }
  }
  __syncthreads();
  // routing index: slot a = a-th smallest active expert, its entries in (t, j) order
  if (wave == 0) {
    const int n = index_lanes(s_ids, f.NK, E, s_pairs, s_slot_e, s_slot_off, s_slot_cnt);
    if (lane == 0) s_meta[0] = n;
  }
  if (blockIdx.x == 0 && threadIdx.x < f.NK) {
    if (f.ids_out) f.ids_out[threadIdx.x] = s_ids[threadIdx.x];
    if (f.gates_out) f.gates_out[threadIdx.x] = s_gates[threadIdx.x];
  }
  __syncthreads();
  // values read from LDS are the same in every lane: readfirstlane makes that
  // visible to the compiler (scalar branches, buffer descriptors in SGPRs)
  const int n_active = uniform(s_meta[0]);
  uint64_t* flags = (uint64_t*)((uint8_t*)f.ctr + kFlagByte);

  if (row == 0) {
    const int a = tk / f.nA, rb = tk - a * f.nA;
    if (a >= n_active) return;            // uniform (also the row's spare workgroups)
    moe_item<FMT, 2, false, true>(m, uniform(s_slot_e[a]), uniform(s_slot_cnt[a]), s_pairs + uniform(s_slot_off[a]), rb,
                                  red);
    __builtin_amdgcn_s_waitcnt(0);        // this thread's h stores have completed
    __syncthreads();
    if (threadIdx.x == 0) flag_store(flags + (size_t)a * f.nA + rb, f.epoch);
    return;
  }

  // output block rt: 16 columns of y for every token
  const int rt = tk;
  float* o_lds = red + FW * 2 * 32 * 4;   // [NK][16]
  // a wave takes slots wave and wave + FW (at most 8 active): int4 and nvfp4
  // request both experts' down weights (the tile's whole K) before the first
  // wait (24 more VGPRs, two waves per SIMD still); int5 and int8, whose
  // kernels would then hold one wave per SIMD, request the second expert's
  // after the first expert is done
  static_assert(2 * FW >= kFusedMaxRows, "two slots per output wave cover every active expert");
  constexpr bool PRE2 = FMT == INT4 || FMT == NVFP4;
  // a slot's h is complete once every row block's flag holds this call's number
  auto wait_slot = [&](int a) {
    const uint64_t* fl = flags + (size_t)a * f.nA;
    uint32_t it = 0;
    for (;;) {
      bool ok = true;
      for (int i = lane; i < f.nA; i += 64) ok &= flag_load(fl + i) == f.epoch;
      if (__all(ok)) break;             // uniform
      if (++it >= kSpinLimit) {
        if (lane == 0) atomicOr(f.ctr + kCtrError, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  // int4 / NVFP4 with both slots and at most four routed pairs between them
  // (always at N = 1): one two-tile k-loop over both experts, whose weights
  // are requested here, before the waits
  const int a1 = wave + FW;
  const bool pair = PRE2 && a1 < n_active && uniform(s_slot_cnt[wave]) + uniform(s_slot_cnt[a1]) <= 4;
  if (pair) {
    const int e0 = uniform(s_slot_e[wave]), e1 = uniform(s_slot_e[a1]);
    const PerTile<2> wq2 = {{make_rsrc(m.wq + (uint64_t)e0 * m.wq_stride, m.wq_bytes),
                             make_rsrc(m.wq + (uint64_t)e1 * m.wq_stride, m.wq_bytes)}};
    const PerTile<2> ws2 = {{make_rsrc(m.ws + (uint64_t)e0 * m.ws_stride, m.ws_bytes),
                             make_rsrc(m.ws + (uint64_t)e1 * m.ws_stride, m.ws_bytes)}};
    const int tile2[2] = {rt, rt};
    Step<FMT, 2, 3> pb[2];
    kloop_start<FMT, 2, 2, 3, true>(pb, wq2, ws2, tile2, m.KS, 0, m.KS, m.hi_offset);
    wait_slot(wave);
    wait_slot(a1);
    down_pair_wave<FMT>(m, wq2, ws2, uniform(s_slot_cnt[wave]), uniform(s_slot_cnt[a1]),
                        s_pairs + uniform(s_slot_off[wave]), s_pairs + uniform(s_slot_off[a1]), rt, o_lds, pb);
  } else {
    Step<FMT, 1, 3> pre[2][2];
    const int tile1[1] = {rt};
    auto start = [&](int i) {
      const int e = uniform(s_slot_e[wave + i * FW]);
      kloop_start<FMT, 1, 2, 3, true>(pre[i], make_rsrc(m.wq + (uint64_t)e * m.wq_stride, m.wq_bytes),
                                      make_rsrc(m.ws + (uint64_t)e * m.ws_stride, m.ws_bytes), tile1, m.KS, 0, m.KS,
                                      m.hi_offset);
    };
    if (wave < n_active) start(0);
    if (PRE2 && wave + FW < n_active) start(1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int a = wave + i * FW;
      if (a >= n_active) break;
      if (i == 1 && !PRE2) start(1);
      auto wait = [&]() { wait_slot(a); };
      down_tile_wave<FMT>(m, uniform(s_slot_e[a]), uniform(s_slot_cnt[a]), s_pairs + uniform(s_slot_off[a]), rt,
                          o_lds, wait, pre[i]);
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < N * 16; o += blockDim.x) {
    const int t = o >> 4, c = o & 15;
    const int col = rt * 16 + c;
    if (col >= f.H) continue;
    float v = f.res ? f.res[(size_t)t * f.H + col] : 0.0f;
    for (int j = 0; j < top_k; ++j) v = fmaf(s_gates[t * top_k + j], o_lds[(t * top_k + j) * 16 + c], v);
    f.y[(size_t)t * f.H + col] = v;
  }
}

}  // namespace qg

using namespace qg;

namespace {

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline size_t up256(size_t v) { return (v + 255) / 256 * 256; }

struct MoeLayout {
  size_t idx_off, h_off, o_off, total;
};

MoeLayout moe_layout(int E, int64_t H, int64_t I, int N, int top_k) {
  const int NK = N * top_k;
  MoeLayout L;
  L.idx_off = 0;
  L.h_off = 0;
  L.o_off = L.h_off + up256((size_t)NK * (size_t)I * 4);
  L.total = L.o_off + up256((size_t)NK * (size_t)H * 4);
  return L;
}

template <int FMT, int NT, bool DOWN>
void launch_moe(const MoeArgs& a, int waves, int slots, hipStream_t stream) {
  constexpr int TO = DOWN ? NT : NT / 2;
  const dim3 grid((unsigned)((a.out_tiles + TO - 1) / TO), (unsigned)slots);
  const size_t lds = (size_t)waves * NT * 32 * 4 * sizeof(float);
  hipLaunchKernelGGL((k_moe_gemv<FMT, NT, DOWN>), grid, dim3(64 * waves), lds, stream, a.ids, a.NK, a.E, a);
}

template <int FMT>
void launch_moe_pair(const MoeArgs& gu, const MoeArgs& dn, int wgu, int wdn, int slots, hipStream_t stream) {
  launch_moe<FMT, 2, false>(gu, wgu, slots, stream);
  launch_moe<FMT, 2, true>(dn, wdn, slots, stream);
}

}  // namespace

extern "C" int qgemv_moe_workspace_bytes(int E, int64_t H, int64_t I, int N, int top_k, size_t* bytes) {
  if (!bytes || E < 1 || H < 1 || I < 1) return QGEMV_EINVAL;
  if (N < 1 || N > 8 || top_k < 1 || top_k > 8) return QGEMV_EUNSUPPORTED;
  *bytes = moe_layout(E, H, I, N, top_k).total;
  return QGEMV_OK;
}

extern "C" int qgemv_moe_index_by(int routine, const int32_t* ids, int N, int top_k, int E, int32_t* counts,
                                  int32_t* offsets, int32_t* pairs, int32_t* active, int32_t* meta,
                                  hipStream_t stream) {
  if (routine != 0 && routine != 1) return QGEMV_EINVAL;
  if (!ids || !counts || !offsets || !pairs || !active || !meta) return QGEMV_EINVAL;
  if (E < 1) return QGEMV_EINVAL;
  if (E > kMaxExperts) return QGEMV_EUNSUPPORTED;
  if (N < 1 || N > 8 || top_k < 1 || top_k > 8) return QGEMV_EUNSUPPORTED;
  if (!al4(ids) || !al4(counts) || !al4(offsets) || !al4(pairs) || !al4(active) || !al4(meta)) return QGEMV_EALIGN;
  if (routine == 0)
    hipLaunchKernelGGL(k_moe_index<0>, dim3(1), dim3(256), 0, stream, ids, N * top_k, E, counts, offsets, pairs,
                       active, meta);
  else
    hipLaunchKernelGGL(k_moe_index<1>, dim3(1), dim3(256), 0, stream, ids, N * top_k, E, counts, offsets, pairs,
                       active, meta);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

extern "C" int qgemv_moe_index(const int32_t* ids, int N, int top_k, int E, int32_t* counts, int32_t* offsets,
                               int32_t* pairs, int32_t* active, int32_t* meta, hipStream_t stream) {
  return qgemv_moe_index_by(0, ids, N, top_k, E, counts, offsets, pairs, active, meta, stream);
}

namespace {

void launch_route(const float* logits, int N, int E, int top_k, int32_t* ids, float* gates, hipStream_t stream) {
  hipLaunchKernelGGL(k_moe_route, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, logits, N, E, top_k, ids, gates);
}

// Shared validation and argument set-up of both MoE entry points (ids and
// gates are checked by the callers). h: two bf16 planes [2][NK][I]; o: fp32
// [NK][H].
int moe_setup(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn, int E, int64_t H,
              int64_t I, const void* x, int top_k, const float* residual, const float* y, int N, void* h, float* o,
              MoeArgs* gu_out, MoeArgs* dn_out, int* wgu_out, int* wdn_out) {
  if (fmt < INT4 || fmt > NVFP4) return QGEMV_EFORMAT;
  if (!wq_gu || !ws_gu || !wq_dn || !ws_dn || !x || !y) return QGEMV_EINVAL;
  if (E < 1 || H < 32 || I < 16) return QGEMV_EINVAL;
  if (E > kMaxExperts) return QGEMV_EUNSUPPORTED;
  if (N < 1 || N > 8 || top_k < 1 || top_k > 8) return QGEMV_EUNSUPPORTED;
  if (H % 32 || I % 32) return QGEMV_EALIGN;
  if (!al16(wq_gu) || !al16(ws_gu) || !al16(wq_dn) || !al16(ws_dn) || !al16(x) || !al4(y) ||
      (residual && !al4(residual)))
    return QGEMV_EALIGN;
  Geom ggu, gdn;
  if (!geom(fmt, 2 * I, H, &ggu) || !geom(fmt, H, I, &gdn)) return QGEMV_EINVAL;
  if ((uint64_t)E * up256(ggu.wq_bytes) >= (1ull << 40)) return QGEMV_EUNSUPPORTED;
  // activation bytes stay below 2^25 (x: N*H bf16; h: N*top_k*I fp32)
  if ((uint64_t)N * H * 2 >= (1ull << 25) || (uint64_t)N * top_k * I * 4 >= (1ull << 25)) return QGEMV_EUNSUPPORTED;
  if ((uint64_t)N * top_k * H * 4 >= (1ull << 31)) return QGEMV_EUNSUPPORTED;
  if (ggu.wq_bytes >= (1ull << 31) || gdn.wq_bytes >= (1ull << 31)) return QGEMV_EUNSUPPORTED;
  const int NK = N * top_k;

  MoeArgs gu;
  gu.wq = (const uint8_t*)wq_gu;
  gu.ws = (const uint8_t*)ws_gu;
  gu.wq_stride = up256(ggu.wq_bytes);
  gu.ws_stride = up256(ggu.ws_bytes);
  gu.wq_bytes = (uint32_t)ggu.wq_bytes;
  gu.ws_bytes = (uint32_t)ggu.ws_bytes;
  gu.hi_offset = (uint32_t)ggu.hi_offset;
  gu.st_offset = (uint32_t)ggu.st_offset;
  gu.in = x;
  gu.in_bytes = (uint32_t)((int64_t)N * H * 2);
  gu.out = (float*)h;
  gu.out_bytes = (uint32_t)((size_t)NK * I * 4);   // two bf16 planes
  gu.ids = nullptr;
  gu.E = E;
  gu.top_k = top_k;
  gu.NK = NK;
  gu.Mout = (int)I;
  gu.K = (int)H;
  gu.KS = (int)ggu.KS;
  gu.G = (int)(H / 32);
  gu.out_tiles = (int)((I + 15) / 16);
  gu.up_tile0 = (int)(I / 16);
  // waves per workgroup (measured on the 128-expert workload): ~4 k-steps per
  // wave while few rows are routed (N * top_k < 32), whole K per wave beyond
  const bool many = NK >= 32;
  const int wgu = many ? 1 : (int)std::min<int64_t>(8, std::max<int64_t>(1, (ggu.KS + 3) / 4));
  gu.ks_per_wave = (int)((ggu.KS + wgu - 1) / wgu);

  MoeArgs dn = gu;
  dn.wq = (const uint8_t*)wq_dn;
  dn.ws = (const uint8_t*)ws_dn;
  dn.wq_stride = up256(gdn.wq_bytes);
  dn.ws_stride = up256(gdn.ws_bytes);
  dn.wq_bytes = (uint32_t)gdn.wq_bytes;
  dn.ws_bytes = (uint32_t)gdn.ws_bytes;
  dn.hi_offset = (uint32_t)gdn.hi_offset;
  dn.st_offset = (uint32_t)gdn.st_offset;
  dn.in = h;
  dn.in_bytes = (uint32_t)((size_t)NK * I * 4);   // two bf16 planes
  dn.out = o;
  dn.out_bytes = (uint32_t)((size_t)NK * H * 4);
  dn.Mout = (int)H;
  dn.K = (int)I;
  dn.KS = (int)gdn.KS;
  dn.G = (int)(I / 32);
  dn.out_tiles = (int)((H + 15) / 16);
  dn.up_tile0 = 0;
  const int wdn = many ? 1 : (int)std::min<int64_t>(8, std::max<int64_t>(1, (gdn.KS + 3) / 4));
  dn.ks_per_wave = (int)((gdn.KS + wdn - 1) / wdn);
  *gu_out = gu;
  *dn_out = dn;
  *wgu_out = wgu;
  *wdn_out = wdn;
  return QGEMV_OK;
}

}  // namespace

extern "C" int qgemv_moe(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn, int E,
                         int64_t H, int64_t I, const void* x, const int32_t* ids, const float* gates, int top_k,
                         const float* residual, float* y, int N, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!ids || !gates) return QGEMV_EINVAL;
  if (!al4(ids) || !al4(gates)) return QGEMV_EALIGN;
  if (!workspace) return QGEMV_EWORKSPACE;
  if (!al16(workspace)) return QGEMV_EALIGN;
  if (E >= 1 && H >= 1 && I >= 1 && N >= 1 && N <= 8 && top_k >= 1 && top_k <= 8 &&
      workspace_bytes < moe_layout(E, H, I, N, top_k).total)
    return QGEMV_EWORKSPACE;
  const MoeLayout L = moe_layout(E, H, I, N, top_k);
  uint8_t* wsp = (uint8_t*)workspace;
  MoeArgs gu, dn;
  int wgu, wdn;
  const int rc = moe_setup(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E, H, I, x, top_k, residual, y, N, wsp + L.h_off,
                           (float*)(wsp + L.o_off), &gu, &dn, &wgu, &wdn);
  if (rc) return rc;
  gu.ids = ids;
  dn.ids = ids;
  const int slots = std::min(E, gu.NK);   // one grid row per active-expert slot
  switch (fmt) {
    case INT4: launch_moe_pair<INT4>(gu, dn, wgu, wdn, slots, stream); break;
    case INT5: launch_moe_pair<INT5>(gu, dn, wgu, wdn, slots, stream); break;
    case INT8: launch_moe_pair<INT8>(gu, dn, wgu, wdn, slots, stream); break;
    default: launch_moe_pair<NVFP4>(gu, dn, wgu, wdn, slots, stream); break;
  }
  const int64_t tot = (int64_t)N * H;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream,
                     (const float*)(wsp + L.o_off), ids, gates, residual, y, N, (int)H, top_k, E);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

// ---- allocation-free MoE (qgemv_moe_noalloc) ---------------------------------
// The h / o scratch of qgemv_moe in a file-scope device array instead of a
// caller workspace. Each GPU the library runs on holds its own copy until the
// process ends; host code never passes the array's name to a kernel (on the
// host it only stands for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QGEMV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QGEMV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QGEMV_OK;
}
}  // namespace

extern "C" int qgemv_moe_noalloc(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn,
                                 int E, int64_t H, int64_t I, const void* x, const int32_t* ids, const float* gates,
                                 int top_k, const float* residual, float* y, int N, hipStream_t stream) {
  if (E < 1 || H < 1 || I < 1) return QGEMV_EINVAL;
  if (N < 1 || N > 8 || top_k < 1 || top_k > 8) return QGEMV_EUNSUPPORTED;
  const size_t need = moe_layout(E, H, I, N, top_k).total;
  if (need > kStaticScratchBytes) return QGEMV_EWORKSPACE;
  void* p = nullptr;
  const int rc = scratch_of_current_device(&p);
  if (rc) return rc;
  return qgemv_moe(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E, H, I, x, ids, gates, top_k, residual, y, N, p,
                   kStaticScratchBytes, stream);
}

extern "C" int qgemv_moe_noalloc_max_bytes(size_t* bytes) {
  if (!bytes) return QGEMV_EINVAL;
  *bytes = kStaticScratchBytes;
  return QGEMV_OK;
}

extern "C" int qgemv_moe_route(const float* logits, int N, int E, int top_k, int32_t* ids, float* gates,
                               hipStream_t stream) {
  if (!logits || !ids || !gates) return QGEMV_EINVAL;
  if (N < 1 || E < 1 || top_k < 1) return QGEMV_EINVAL;
  if (top_k > 64 || top_k > E || E > kMaxExperts || (int64_t)N * E >= (1ll << 31)) return QGEMV_EUNSUPPORTED;
  if (!al4(logits) || !al4(ids) || !al4(gates)) return QGEMV_EALIGN;
  launch_route(logits, N, E, top_k, ids, gates, stream);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}

namespace {

struct FusedLayout {
  size_t ctr_bytes, route_off, h_off, o_off, total;
};

// The error word and the item flags first (their size depends on I only,
// so calls with the same I may share a workspace whatever their N, E, H),
// then ids and weights of the routing (when the caller passes no buffers for
// them), h and o.
FusedLayout fused_layout(int64_t H, int64_t I, int N, int top_k) {
  const size_t NK = (size_t)N * top_k;
  const size_t nA = (size_t)((I + 15) / 16);
  FusedLayout L;
  L.ctr_bytes = up256((size_t)kFlagByte + (size_t)kFusedMaxRows * nA * 8);
  L.route_off = L.ctr_bytes;
  L.h_off = L.route_off + 512;            // 64 ids + 64 weights
  L.o_off = L.h_off + up256(NK * (size_t)I * 4);
  L.total = L.o_off + up256(NK * (size_t)H * 4);
  return L;
}
std::atomic<uint64_t> g_fused_epoch{0};
template <int FMT>
hipError_t launch_fused(const MoeFusedArgs& f, hipStream_t stream) {
  constexpr int FW = kFusedWaves;
  const size_t lds = (size_t)(FW * 2 * 32 * 4 + kFusedMaxRows * 16) * sizeof(float);
  // row 0: one workgroup per (slot, gate/up row block); row 1: one per output
  // block. Linear workgroup ids run along x first, so every output
  // workgroup comes after every gate/up workgroup in dispatch order.
  const unsigned gx = (unsigned)std::max(f.slots * f.nA, f.nB);
  hipLaunchKernelGGL(k_moe_fused<FMT>, dim3(gx, 2), dim3(64 * FW), lds, stream, f.logits, f.E, f.top_k, f.N, f);
  return hipGetLastError();
}
}  // namespace

extern "C" int qgemv_moe_fused_workspace_bytes(int E, int64_t H, int64_t I, int N, int top_k, size_t* bytes) {
  if (!bytes || E < 1 || H < 1 || I < 1) return QGEMV_EINVAL;
  if (N < 1 || N > 8 || top_k < 1 || top_k > 8) return QGEMV_EUNSUPPORTED;
  *bytes = fused_layout(H, I, N, top_k).total;
  return QGEMV_OK;
}

extern "C" int qgemv_moe_fused(int fmt, const void* wq_gu, const void* ws_gu, const void* wq_dn, const void* ws_dn,
                               int E, int64_t H, int64_t I, const void* x, const float* logits, int top_k,
                               const float* residual, float* y, int N, int32_t* ids_out, float* gates_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!logits) return QGEMV_EINVAL;
  if (!al4(logits) || (ids_out && !al4(ids_out)) || (gates_out && !al4(gates_out))) return QGEMV_EALIGN;
  if (!workspace) return QGEMV_EWORKSPACE;
  if (!al16(workspace)) return QGEMV_EALIGN;
  if (E >= 1 && top_k > E) return QGEMV_EUNSUPPORTED;
  if (E >= 1 && H >= 1 && I >= 1 && N >= 1 && N <= 8 && top_k >= 1 && top_k <= 8 &&
      workspace_bytes < fused_layout(H, I, N, top_k).total)
    return QGEMV_EWORKSPACE;
  const FusedLayout L = fused_layout(H, I, N, top_k);
  uint8_t* wsp = (uint8_t*)workspace;
  MoeFusedArgs f;
  int wgu, wdn;
  const int rc = moe_setup(fmt, wq_gu, ws_gu, wq_dn, ws_dn, E, H, I, x, top_k, residual, y, N, wsp + L.h_off,
                           (float*)(wsp + L.o_off), &f.g[0], &f.g[1], &wgu, &wdn);
  if (rc) return rc;
  f.logits = logits;
  f.res = residual;
  f.y = y;
  f.ctr = (uint32_t*)wsp;
  f.N = N;
  f.H = (int)H;
  f.E = E;
  f.top_k = top_k;
  f.NK = N * top_k;
  f.slots = std::min(E, f.NK);
  if (f.NK > kFusedMaxRows) {
    // more routed rows: the router in its own launch, then the three launches
    // of qgemv_moe on its ids and weights (measured faster from 16 rows: the
    // single launch's chain of dependent memory round trips outweighs the
    // launches it saves)
    int32_t* ids = ids_out ? ids_out : (int32_t*)(wsp + L.route_off);
    float* gates = gates_out ? gates_out : (float*)(wsp + L.route_off + 256);
    launch_route(logits, N, E, top_k, ids, gates, stream);
    f.g[0].ids = ids;
    f.g[1].ids = ids;
    switch (fmt) {
      case INT4: launch_moe_pair<INT4>(f.g[0], f.g[1], wgu, wdn, f.slots, stream); break;
      case INT5: launch_moe_pair<INT5>(f.g[0], f.g[1], wgu, wdn, f.slots, stream); break;
      case INT8: launch_moe_pair<INT8>(f.g[0], f.g[1], wgu, wdn, f.slots, stream); break;
      default: launch_moe_pair<NVFP4>(f.g[0], f.g[1], wgu, wdn, f.slots, stream); break;
    }
    const int64_t tot = (int64_t)N * H;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(wsp + L.o_off), ids, gates, residual, y, N, (int)H, top_k, E);
    return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
  }
  // few routed rows: one launch; gate/up items split K over its waves
  f.g[0].ks_per_wave = (f.g[0].KS + kFusedWaves - 1) / kFusedWaves;
  f.epoch = g_fused_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  f.ids_out = ids_out;
  f.gates_out = gates_out;
  f.nA = f.g[0].out_tiles;                  // one gate tile and its up tile per item
  f.nB = f.g[1].out_tiles;                  // 16 output columns per item
  hipError_t e;
  switch (fmt) {
    case INT4: e = launch_fused<INT4>(f, stream); break;
    case INT5: e = launch_fused<INT5>(f, stream); break;
    case INT8: e = launch_fused<INT8>(f, stream); break;
    default: e = launch_fused<NVFP4>(f, stream); break;
  }
  return e == hipSuccess ? QGEMV_OK : QGEMV_EHIP;
}
