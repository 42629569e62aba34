// grouped_kernels.h -- the MoE layer for B > 1 tokens, with the tokens grouped
// by expert: every weight row of the layer (router, shared expert, each
// distinct routed expert) is read from HBM once per layer-step and applied to
// all the tokens that use it. Included by kernels_q4.hip / kernels_q2.hip after
// layer_kernels.h, which instantiate group_b<BITS>.
//
// Five launches:
//   g1  router logits and sigmoid(g . x) of every token, shared expert
//       gate/up + SwiGLU of every token (weights in registers, the tokens'
//       x vectors staged through LDS kTokChunk at a time)
//   g2r one workgroup: top-K of every token, then the distinct experts in
//       order of first use and, for each, the ascending list of the slots
//       (token t, choice k; slot = t*K + k) routed to it
//   g2  routed gate/up + SwiGLU by (distinct expert, block of rows) for the
//       expert's slots; the shared expert's down for every token
//   g3  routed down by (distinct expert, block of rows): per slot, w * (D h)
//   g4  out = residual + the K per-slot outputs in slot order + sigma * shared
#pragma once

#include "layer_kernels.h"

namespace fmoe {
namespace dev {

constexpr int kTokChunk = 2;   // hidden-wide vectors staged in LDS at a time
// inter-wide vectors staged in LDS at a time (NGI groups each): at most 128 groups
template <int NGI>
constexpr int hchunk() { return NGI >= 64 ? 2 : NGI >= 32 ? 4 : 8; }
constexpr int kG2Iters = 2;    // gate/up pair iterations per wavefront per work item
constexpr int kG3Iters = 4;    // down row iterations per wavefront per work item
constexpr int kG2DownIters = 4;  // shared down row iterations per wavefront
constexpr int kRouteThreads = 1024;
constexpr int kMaxSlots = kMaxTokens * kMaxTopK;
static_assert(kMaxSlots <= kRouteThreads, "one routing thread per slot");


// Stage a hidden-wide (or inter-wide) vector through the generic helper of the
// one-token kernels, with or without the sum of squares.
template <int NG>
__device__ __forceinline__ void stage_tok(const float *src, float *lds, float *part, bool sumsq) {
  if (sumsq)
    stage_vec<NG, true>(src, lds, part);
  else
    stage_vec<NG, false>(src, lds, part);
}

// g1: router rows (one fp32 row per wavefront; row E is the gate vector) or
// shared-expert gate/up pairs, for every token.
template <int BITS, int NGH>
__global__ __launch_bounds__(kBlock) void k_g1(const GroupArgs a) {
  constexpr int NT = NGH / 4;
  constexpr int H = NGH * kGroup;
  constexpr int RPIH = kWave / NGH;
  constexpr int X4 = (NGH * 16 + kBlock - 1) / kBlock;
  __shared__ float xl[kTokChunk][NGH * kXPad];
  __shared__ float part[kTokChunk][kWavesPerBlock];
  const int lane = lane_id();
  const bool rms = a.rms_eps >= 0.f;
  const bool router = (int)blockIdx.x < a.n_router_blocks;
  const int n_rows = a.E + (a.gvec ? 1 : 0);
  const int row = blockIdx.x * kWavesPerBlock + wave_in_block();
  const int pair0 = ((blockIdx.x - a.n_router_blocks) * kWavesPerBlock + wave_in_block()) * RPIH;
  // token 0's x is requested before the weights (memory counters complete in order)
  Staged<X4> xst;
  stage_load(a.x, NGH * 16, xst);
  float4 wr[NT];
  PairLoads<BITS, NGH, 1> P;
  if (router) {
    const int rr = min(row, n_rows - 1);
    const float *src = rr == a.E ? a.gvec : a.router + (size_t)rr * H;
#pragma unroll
    for (int t = 0; t < NT; ++t) wr[t] = reinterpret_cast<const float4 *>(src)[lane + 64 * t];
  } else if (pair0 < a.I) {
    P.issue(a.shared, pair0);
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int t0 = 0; t0 < a.B; t0 += kTokChunk) {
    const int nt = min(kTokChunk, a.B - t0);
    if (t0 > 0) __syncthreads();  // the previous chunk's reads of xl are done
    for (int j = 0; j < nt; ++j) {
      if (t0 + j == 0) {
        if (rms)
          stage_store<X4, true>(xst, NGH * 16, xl[0], part[0]);
        else
          stage_store<X4, false>(xst, NGH * 16, xl[0], part[0]);
      } else {
        stage_tok<NGH>(a.x + (size_t)(t0 + j) * H, xl[j], part[j], rms);
      }
    }
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const int t = t0 + j;
      const float inv = rms ? rms_inv(part[j], H, a.rms_eps) : 1.f;
      if (router) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          const float4 xv = *reinterpret_cast<const float4 *>(&xl[j][lds_index(4 * lane + 256 * q)]);
          acc = fmaf(wr[q].x, xv.x * inv, acc);
          acc = fmaf(wr[q].y, xv.y * inv, acc);
          acc = fmaf(wr[q].z, xv.z * inv, acc);
          acc = fmaf(wr[q].w, xv.w * inv, acc);
        }
        const float d = seg_reduce<kWave>(acc);
        if (lane == kWave - 1 && row < n_rows) {
          if (row == a.E)
            a.sigma[t] = 1.f / (1.f + expf(-d));
          else
            a.logits[(size_t)t * a.E + row] = d;
        }
      } else if (pair0 < a.I) {
        XSlice xs;
        read_slice(xl[j], lane & (NGH - 1), inv, xs);
        P.finish(xs, a.h_shared + (size_t)t * a.I, pair0);
      }
    }
  }
}

// g2r: one workgroup of kRouteThreads. Top-K of each token (one wavefront per
// token), then the grouping, deterministic whatever the thread timing:
//  - first[e] = the lowest slot routed to expert e (an atomic minimum);
//  - the slots with first[e] == slot lead their expert; the leaders, in slot
//    order, number the distinct experts 0..D-1;
//  - every slot's position in its expert's list = the number of lower slots
//    routed to the same expert, so each list is in ascending slot order.
template <int BITS>  // (instantiated per bit width, like the rest of the layer)
__global__ __launch_bounds__(kRouteThreads) void k_g2r(const GroupArgs a) {
  constexpr int NW = kRouteThreads / kWave;
  __shared__ int first[kMaxExperts];
  __shared__ int sidx[kMaxSlots];
  __shared__ int rank_of[kMaxSlots];
  __shared__ int cnt[kMaxSlots];
  __shared__ int off[kMaxSlots + 1];
  __shared__ int wsum[NW];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int S = a.B * a.K;
  for (int t = wave; t < a.B; t += NW) {
    int idx[kMaxTopK];
    float w[kMaxTopK];
    wave_topk_lds(a.logits + (size_t)t * a.E, a.E, a.K, idx, w);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j == lane && j < a.K) {
        const int s = t * a.K + j;
        a.idx[s] = idx[j];
        a.w[s] = w[j];
        if (a.out_idx) a.out_idx[s] = idx[j];
        if (a.out_w) a.out_w[s] = w[j];
        sidx[s] = idx[j];
      }
  }
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) first[e] = 0x7FFFFFFF;
  __syncthreads();
  const int s = threadIdx.x;
  if (s < S) atomicMin(&first[sidx[s]], s);
  __syncthreads();
  const bool lead = s < S && first[sidx[s]] == s;
  const unsigned long long bl = __ballot(lead);
  if (lane == 0) wsum[wave] = __popcll(bl);
  __syncthreads();
  int before = 0, D = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    before += v < wave ? wsum[v] : 0;
    D += wsum[v];
  }
  const int rank = before + __popcll(bl & ((1ull << lane) - 1ull));
  if (lead) {
    rank_of[s] = rank;
    cnt[rank] = 0;
  }
  __syncthreads();
  int r = 0, pos = 0;
  if (s < S) {
    const int e = sidx[s];
    r = rank_of[first[e]];
    for (int q = first[e]; q < s; ++q) pos += sidx[q] == e;
    atomicAdd(&cnt[r], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0;
    for (int q = 0; q < D; ++q) {
      off[q] = o;
      o += cnt[q];
    }
    off[D] = o;
  }
  __syncthreads();
  int32_t *G = a.groups;
  if (threadIdx.x == 0) G[0] = D;
  if (lead) G[1 + rank] = sidx[s];
  if ((int)threadIdx.x <= D) G[1 + S + threadIdx.x] = off[threadIdx.x];
  if (s < S) G[1 + S + (S + 1) + off[r] + pos] = s;
}

// g2: routed gate/up by work item (distinct expert d, block of pair rows), and
// the shared expert's down projection for every token (scaled by its sigma).
template <int BITS, int NGH, int NGI>
__global__ __launch_bounds__(kBlock) void k_g2(const GroupArgs a) {
  constexpr int H = NGH * kGroup;
  constexpr int RPIH = kWave / NGH;
  constexpr int HC = hchunk<NGI>();
  constexpr int BUF = (kTokChunk * NGH > HC * NGI ? kTokChunk * NGH : HC * NGI) * kXPad;
  __shared__ float buf[BUF];
  __shared__ float part[kTokChunk][kWavesPerBlock];
  const int lane = lane_id();
  if ((int)blockIdx.x < a.n_g2_routed_blocks) {
    const bool rms = a.rms_eps >= 0.f;
    const int32_t *G = a.groups;
    const int S = a.B * a.K;
    const int D = G[0];
    constexpr int kPairsPerItem = kWavesPerBlock * kG2Iters * RPIH;
    const int per = a.I / kPairsPerItem;
    for (int item = blockIdx.x; item < D * per; item += a.n_g2_routed_blocks) {
      const int d = item / per;
      const int pair0 = ((item - d * per) * kWavesPerBlock + wave_in_block()) * kG2Iters * RPIH;
      const int e = G[1 + d];
      const int q0 = G[1 + S + d], q1 = G[1 + S + d + 1];
      const int32_t *slots = G + 1 + S + (S + 1);
      PairLoads<BITS, NGH, kG2Iters> P;
      P.issue(a.bank + (size_t)e * a.stride, pair0);
      for (int c = q0; c < q1; c += kTokChunk) {
        const int nt = min(kTokChunk, q1 - c);
        __syncthreads();  // buf is free
        for (int j = 0; j < nt; ++j)
          stage_tok<NGH>(a.x + (size_t)(slots[c + j] / a.K) * H, buf + j * NGH * kXPad, part[j], rms);
        __syncthreads();
        for (int j = 0; j < nt; ++j) {
          XSlice xs;
          read_slice(buf + j * NGH * kXPad, lane & (NGH - 1), rms ? rms_inv(part[j], H, a.rms_eps) : 1.f, xs);
          P.finish(xs, a.h_routed + (size_t)slots[c + j] * a.I, pair0);
        }
      }
    }
    return;
  }
  const int wv = (blockIdx.x - a.n_g2_routed_blocks) * kWavesPerBlock + wave_in_block();
  const int row0 = wv * kG2DownIters * (kWave / NGI);
  RowLoads<BITS, NGI, kG2DownIters> R;
  if (row0 < a.H) R.issue(a.shared + a.gu_bytes, a.H, row0);
  for (int t0 = 0; t0 < a.B; t0 += HC) {
    const int nt = min(HC, a.B - t0);
    if (t0 > 0) __syncthreads();
    for (int j = 0; j < nt; ++j)
      stage_vec<NGI, false>(a.h_shared + (size_t)(t0 + j) * a.I, buf + j * NGI * kXPad, nullptr);
    __syncthreads();
    if (row0 < a.H) {
      for (int j = 0; j < nt; ++j) {
        XSlice xs;
        read_slice(buf + j * NGI * kXPad, lane & (NGI - 1), 1.f, xs);
        R.finish(xs, a.d_shared + (size_t)(t0 + j) * a.H, a.H, row0, a.sigma[t0 + j]);
      }
    }
  }
}

// g3: routed down by work item (distinct expert d, block of rows): for each of
// the expert's slots s, partial[s][row] = w[s] * (down_row . h[s]).
template <int BITS, int NGI>
__global__ __launch_bounds__(kBlock) void k_g3(const GroupArgs a) {
  constexpr int RPII = kWave / NGI;
  constexpr int kRowsPerItem = kWavesPerBlock * kG3Iters * RPII;
  constexpr int HC = hchunk<NGI>();
  __shared__ float buf[HC * NGI * kXPad];
  const int lane = lane_id();
  const int32_t *G = a.groups;
  const int S = a.B * a.K;
  const int D = G[0];
  const int per = (a.H + kRowsPerItem - 1) / kRowsPerItem;
  const int32_t *slots = G + 1 + S + (S + 1);
  for (int item = blockIdx.x; item < D * per; item += gridDim.x) {
    const int d = item / per;
    const int row0 = ((item - d * per) * kWavesPerBlock + wave_in_block()) * kG3Iters * RPII;
    const int e = G[1 + d];
    const int q0 = G[1 + S + d], q1 = G[1 + S + d + 1];
    RowLoads<BITS, NGI, kG3Iters> R;
    if (row0 < a.H) R.issue(a.bank + (size_t)e * a.stride + a.gu_bytes, a.H, row0);
    for (int c = q0; c < q1; c += HC) {
      const int nt = min(HC, q1 - c);
      __syncthreads();
      for (int j = 0; j < nt; ++j)
        stage_vec<NGI, false>(a.h_routed + (size_t)slots[c + j] * a.I, buf + j * NGI * kXPad, nullptr);
      __syncthreads();
      if (row0 < a.H) {
        for (int j = 0; j < nt; ++j) {
          const int s = slots[c + j];
          XSlice xs;
          read_slice(buf + j * NGI * kXPad, lane & (NGI - 1), 1.f, xs);
          R.finish(xs, a.partial + (size_t)s * a.H, a.H, row0, a.w[s]);
        }
      }
    }
  }
}

// g4: out[t] = residual[t] + sum_k partial[t*K + k] (k ascending) + d_shared[t]
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_g4(const GroupArgs a) {
  const int f = blockIdx.x * kBlock + threadIdx.x;  // float4 index into [B][H]
  const int h4 = a.H / 4;
  if (f >= a.B * h4) return;
  const int t = f / h4, i = f - t * h4;
  float4 o = reinterpret_cast<const float4 *>(a.residual)[f];
  for (int k = 0; k < a.K; ++k) {
    const float4 p = reinterpret_cast<const float4 *>(a.partial)[(size_t)(t * a.K + k) * h4 + i];
    o.x += p.x;
    o.y += p.y;
    o.z += p.z;
    o.w += p.w;
  }
  if (a.shared) {
    const float4 q = reinterpret_cast<const float4 *>(a.d_shared)[f];
    o.x += q.x;
    o.y += q.y;
    o.z += q.z;
    o.w += q.w;
  }
  reinterpret_cast<float4 *>(a.out)[f] = o;
}

// Workgroup caps of the grid-stride kernels (a few per CU).
constexpr int kG2Blocks = 512;
constexpr int kG3Blocks = 512;

template <int BITS>
struct GroupDispatch {
  template <int NGH, int NGI>
  static hipError_t layer(GroupArgs a, hipStream_t s, int phases) {
    constexpr int RPIH = kWave / NGH, RPII = kWave / NGI;
    const bool sh = a.shared != nullptr;
    const int S = a.B * a.K;
    const int dmax = S < a.E ? S : a.E;
    a.n_router_blocks = blocks_for(a.E + (sh ? 1 : 0));
    const int n1s = sh ? blocks_for(a.I / RPIH) : 0;
    const long items2 = (long)dmax * (a.I / (kWavesPerBlock * kG2Iters * RPIH));
    a.n_g2_routed_blocks = (int)(items2 < kG2Blocks ? items2 : kG2Blocks);
    const int n2s = sh ? blocks_for((a.H / RPII + kG2DownIters - 1) / kG2DownIters) : 0;
    const int rows3 = kWavesPerBlock * kG3Iters * RPII;
    const long items3 = (long)dmax * ((a.H + rows3 - 1) / rows3);
    const int n3 = (int)(items3 < kG3Blocks ? items3 : kG3Blocks);
    const int n4 = (a.B * (a.H / 4) + kBlock - 1) / kBlock;
    if (phases & 1) hipLaunchKernelGGL((k_g1<BITS, NGH>), dim3(a.n_router_blocks + n1s), dim3(kBlock), 0, s, a);
    if (phases & 2) {
      hipLaunchKernelGGL(k_g2r<BITS>, dim3(1), dim3(kRouteThreads), 0, s, a);
      hipLaunchKernelGGL((k_g2<BITS, NGH, NGI>), dim3(a.n_g2_routed_blocks + n2s), dim3(kBlock), 0, s, a);
    }
    if (phases & 4) {
      hipLaunchKernelGGL((k_g3<BITS, NGI>), dim3(n3), dim3(kBlock), 0, s, a);
      hipLaunchKernelGGL(k_g4<BITS>, dim3(n4), dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
  }

  template <int NGH>
  static hipError_t layer_h(const GroupArgs &a, hipStream_t s, int phases) {
    switch (a.I / kGroup) {
      case 4: return layer<NGH, 4>(a, s, phases);
      case 8: return layer<NGH, 8>(a, s, phases);
      case 16: return layer<NGH, 16>(a, s, phases);
      case 32: return layer<NGH, 32>(a, s, phases);
      case 64: return layer<NGH, 64>(a, s, phases);
      default: return hipErrorInvalidValue;
    }
  }
};

template <int BITS>
hipError_t group_b(const GroupArgs &a, hipStream_t s, int phases) {
  FMOE_NG_SWITCH(a.H / kGroup, GroupDispatch<BITS>::template layer_h, a, s, phases)
}

}  // namespace dev
}  // namespace fmoe
