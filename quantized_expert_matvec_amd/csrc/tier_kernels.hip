// tier_kernels.hip -- the host-memory expert tier with its policy on the GPU: the
// cache's least-recently-used plan of one layer call and the copies it needs, run
// as two kernels after the routing, so that a tiered layer needs no host
// synchronisation (and can be captured in a graph).
//
// The pages stream the chosen experts from SSD and let the operating system's page
// cache keep the recently used ones ("397B MoE en MacBook: Motor Flash-MoE a 4,4
// t/s", section "1. Streaming de expertos desde SSD + 'Confia en el SO'";
// "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook Pro mit
// reinem C/Metal", section "SSD-Experten-Streaming"). Here the slow tier is pinned
// host memory, the fast one a set of HBM slots, and the policy the one of the
// host-side bookkeeping (expert_cache.h), evaluated on the device: a call's
// distinct experts in ascending id; a hit refreshes its slot; a miss takes the
// first empty slot, else the least recently used slot the call does not hold,
// ties to the lower slot.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"
#include "layout.h"

namespace fmoe {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
static_assert(kMaxExperts <= kPlanThreads, "one expert per thread in the scans");

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long u = __shfl_xor(v, o);
    v = u < v ? u : v;
  }
  return v;
}

// Exclusive prefix sum of v over the workgroup (thread order); *total the sum.
__device__ __forceinline__ int block_scan_excl(int v, int *wt, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    base += i < w ? wt[i] : 0;
    tot += wt[i];
  }
  total = tot;
  __syncthreads();  // (wt reused by the next scan)
  return base + x - v;
}

// The plan of one call, by one workgroup. Slots the call holds (its hits, then its
// victims) are marked in an LDS bitmap, so that nothing the kernel writes to the
// global state is read back by it.
__global__ __launch_bounds__(kPlanThreads) void k_tier_plan(const TierPlanArgs a) {
  __shared__ int present[kMaxExperts];
  __shared__ int exl[kMaxExperts];      // the distinct experts, ascending
  __shared__ int slot_of[kMaxExperts];  // slot of each chosen expert (-1: a miss, until placed)
  __shared__ int miss_i[kMaxExperts];   // call index of the m-th miss
  __shared__ uint32_t held[kMaxTierSlots / 32];
  __shared__ int wt[kPlanWaves];
  __shared__ unsigned long long red[kPlanWaves];
  const int tid = threadIdx.x;
  for (int e = tid; e < kMaxExperts; e += kPlanThreads) {
    present[e] = 0;
    slot_of[e] = -1;
  }
  for (int i = tid; i < (a.n_slots + 31) / 32; i += kPlanThreads) held[i] = 0u;
  __syncthreads();
  for (int s = tid; s < a.S; s += kPlanThreads) {
    const int e = a.idx[s];
    if (e >= 0 && e < a.E) present[e] = 1;
  }
  __syncthreads();
  int n;
  {
    const int v = tid < a.E ? present[tid] : 0;
    const int pos = block_scan_excl(v, wt, n);
    if (v) exl[pos] = tid;
  }
  const uint64_t call = a.hdr->call + 1, clock0 = a.hdr->clock;
  // lookups: the slots that hold one of the call's experts are the call's
  for (int p = tid; p < a.n_slots; p += kPlanThreads) {
    const int64_t k = a.key[p];
    if (k >= 0 && (int)(k >> 32) == a.layer) {
      const int e = (int)(k & 0xFFFFFFFF);
      if (e < a.E && present[e]) {
        slot_of[e] = p;
        atomicOr(&held[p >> 5], 1u << (p & 31));
      }
    }
  }
  __syncthreads();
  // the misses, ranked in the call's order; the hits' slots refreshed in that order
  int M;
  {
    const bool live = tid < n;
    const bool miss = live && slot_of[exl[tid]] < 0;
    const int r = block_scan_excl(miss ? 1 : 0, wt, M);
    if (miss) miss_i[r] = tid;
    if (live && !miss) a.last[slot_of[exl[tid]]] = clock0 + (uint64_t)tid + 1;
  }
  __syncthreads();
  // one victim per miss, in order: the least candidate under (empty slots by index;
  // then the slots the call does not hold, by last use, then index)
  int njobs = 0;  // (thread 0's count of the copies)
  for (int m = 0; m < M; ++m) {  // (uniform)
    unsigned long long best = ~0ull;
    for (int p = tid; p < a.n_slots; p += kPlanThreads) {
      if (held[p >> 5] & (1u << (p & 31))) continue;
      const int64_t k = a.key[p];
      const unsigned long long c =
          k < 0 ? (unsigned long long)p : (1ull << 63) | (a.last[p] << 16) | (unsigned long long)p;
      best = c < best ? c : best;
    }
    best = wave_min_u64(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long b = red[0];
#pragma unroll
      for (int w = 1; w < kPlanWaves; ++w) b = red[w] < b ? red[w] : b;
      const int v = (int)(b & 0xFFFF);
      // (a candidate always exists: the caller checked that every call's experts fit;
      // were there none, the expert would get no slot and no copy)
      if (b != ~0ull && v < a.n_slots) {
        const int i = miss_i[m], e = exl[i];
        a.key[v] = ((int64_t)a.layer << 32) | (uint32_t)e;
        a.last[v] = clock0 + (uint64_t)i + 1;
        held[v >> 5] |= 1u << (v & 31);
        slot_of[e] = v;
        a.jobs[2 * njobs] = v;
        a.jobs[2 * njobs + 1] = e;
        ++njobs;
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < n; i += kPlanThreads) {
    const int e = exl[i];
    a.table[e] = a.slots + (size_t)max(slot_of[e], 0) * a.stride;
  }
  if (tid == 0) {
    a.hdr->call = call;
    a.hdr->clock = clock0 + (uint64_t)n;
    a.hdr->lookups += n;
    a.hdr->hits += n - M;
    a.hdr->misses += M;
    a.hdr->bytes += (int64_t)M * (int64_t)a.stride;
    a.hdr->njobs = njobs;
  }
}

constexpr int kCopyThreads = 256;
constexpr int kCopyBlocks = 512;
constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per thread

// The planned copies: every workgroup takes a strided share of each blob, reading
// the pinned host bank over the bus and writing the slot.
__global__ __launch_bounds__(kCopyThreads) void k_tier_copy(const TierHdr *hdr, const int32_t *jobs,
                                                            const uint8_t *host_bank, uint8_t *slots,
                                                            size_t stride) {
  const int M = hdr->njobs;
  const size_t n16 = stride / 16;
  const size_t step = (size_t)gridDim.x * kCopyThreads;
  for (int j = 0; j < M; ++j) {
    const uint4 *src = reinterpret_cast<const uint4 *>(host_bank + (size_t)jobs[2 * j + 1] * stride);
    uint4 *dst = reinterpret_cast<uint4 *>(slots + (size_t)jobs[2 * j] * stride);
    for (size_t u = (size_t)blockIdx.x * kCopyThreads + threadIdx.x; u < n16; u += kCopyUnroll * step) {
      uint4 v[kCopyUnroll];
#pragma unroll
      for (int k = 0; k < kCopyUnroll; ++k) v[k] = src[min(u + k * step, n16 - 1)];
#pragma unroll
      for (int k = 0; k < kCopyUnroll; ++k)
        if (u + k * step < n16) dst[u + k * step] = v[k];
    }
  }
}

__global__ __launch_bounds__(256) void k_tier_init(TierHdr *hdr, int64_t *key, int n_slots) {
  for (int p = blockIdx.x * 256 + threadIdx.x; p < n_slots; p += gridDim.x * 256) key[p] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *hdr = TierHdr{};
}

}  // namespace

hipError_t launch_tier_init(TierHdr *hdr, int64_t *key, int n_slots, hipStream_t s) {
  hipLaunchKernelGGL(k_tier_init, dim3(std::max(1, std::min(256, (n_slots + 255) / 256))), dim3(256), 0, s, hdr, key,
                     n_slots);
  return hipGetLastError();
}

hipError_t launch_tier_plan(const TierPlanArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_tier_plan, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tier_copy(const TierHdr *hdr, const int32_t *jobs, const uint8_t *host_bank, uint8_t *slots,
                            size_t stride, hipStream_t s) {
  hipLaunchKernelGGL(k_tier_copy, dim3(kCopyBlocks), dim3(kCopyThreads), 0, s, hdr, jobs, host_bank, slots, stride);
  return hipGetLastError();
}

}  // namespace fmoe
