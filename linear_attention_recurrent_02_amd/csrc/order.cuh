// order.cuh -- workgroup-level helpers: an exclusive scan, and the
// slot-ordered traversal of a request batch.
//
// Why an order: a decode launch streams every request's state tile once.
// Measured on MI355X, when the requests' slots are a random permutation of
// the pool (1 MiB slots), the state stream runs ~5-7% slower than when the
// workgroups that run at the same time touch neighbouring slots; permuting at
// 4 MiB granularity or coarser costs nothing.  So the persistent decode kernel
// walks requests in ascending write-slot order.  Every workgroup builds the
// same order in LDS from the write-slot array (a bitmap of used slots plus a
// prefix popcount: O(B / threads) work, no extra launch, no device scratch).
// Results do not depend on the order: requests are independent.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Slot ordering is used when the batch's order and the slot bitmap fit in a
// few KiB of LDS; larger batches or pools run in request order.
constexpr int kOrderMaxB = 4096;
constexpr int64_t kOrderMaxSlots = 32768;

// Exclusive prefix sum of x over the NT threads of the workgroup (thread
// order); `total` receives the sum over all threads.  `wsum` is LDS of at
// least NT/64 ints.  Contains two barriers; every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int *wsum, int &total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wsum[w];
    base += (w < wave) ? s : 0;
    tot += s;
  }
  total = tot;
  __syncthreads();
  return base + v - x;
}

// LDS needed by build_slot_order for B requests over n_slots slots.
__host__ __device__ constexpr size_t slot_order_lds_bytes(int B, int64_t n_slots, int NT) {
  return sizeof(int) * ((size_t)B + 2 * (size_t)((n_slots + 31) / 32) + (size_t)(NT / 64) + 1);
}

// order[0..B) <- request indices sorted by ascending write slot, followed by
// the requests whose write slot is -1 or out of range, in request order.  If
// two requests name the same write slot (a caller-contract violation) the
// order is the identity, so every request is still visited exactly once.
// `lds` must hold slot_order_lds_bytes(B, n_slots, NT) bytes.  Every thread
// must call it; ends with a barrier.
template <int NT>
__device__ void build_slot_order(const int32_t *__restrict__ write_slot, int B, int64_t n_slots,
                                 int *lds) {
  constexpr int NW = NT / 64;
  const int W = (int)((n_slots + 31) / 32);
  int *order = lds;
  uint32_t *bm = reinterpret_cast<uint32_t *>(lds + B);
  int *wpre = lds + B + W;
  int *wsum = lds + B + 2 * W;
  int *dup = wsum + NW;
  const int tid = threadIdx.x;

  for (int w = tid; w < W; w += NT) bm[w] = 0u;
  if (tid == 0) *dup = 0;
  __syncthreads();

  // each thread owns a contiguous run of requests (so the tail keeps request order)
  const int C = (B + NT - 1) / NT;
  const int r0 = min(B, tid * C), r1 = min(B, r0 + C);
  int tail_mine = 0;
  for (int r = r0; r < r1; ++r) {
    const int64_t s = write_slot[r];
    if (s >= 0 && s < n_slots) {
      const uint32_t bit = 1u << (s & 31);
      if (atomicOr(&bm[s >> 5], bit) & bit) *dup = 1;
    } else {
      ++tail_mine;
    }
  }
  __syncthreads();
  const bool collide = *dup != 0;

  // exclusive prefix popcount over the bitmap words (contiguous runs per thread)
  const int CW = (W + NT - 1) / NT;
  const int w0 = min(W, tid * CW), w1 = min(W, w0 + CW);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int n_valid;
  int run = block_exclusive_scan<NT>(cnt, wsum, n_valid);
  for (int w = w0; w < w1; ++w) {
    wpre[w] = run;
    run += __popc(bm[w]);
  }
  int n_tail;
  int tail = block_exclusive_scan<NT>(tail_mine, wsum, n_tail);  // barriers publish wpre too

  for (int r = r0; r < r1; ++r) {
    const int64_t s = write_slot[r];
    int rank;
    if (collide) {
      rank = r;
    } else if (s >= 0 && s < n_slots) {
      rank = wpre[s >> 5] + __popc(bm[s >> 5] & ((1u << (s & 31)) - 1u));
    } else {
      rank = n_valid + tail++;
    }
    order[rank] = r;
  }
  __syncthreads();
}

}  // namespace gdn
