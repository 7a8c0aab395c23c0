// Scheduling pre-pass for the block-sparse FP8 prefill, gfx950.
//
// "Quant Block Sparse Attention" ("Sparse indices & PA page table") splits the
// (batch, query head, query block) tasks between cores with a metadata operator
// that reads the sparse workload on the device, on the same stream as the
// attention, so that the host never reads it back.  Here the GPU's workgroup
// dispatcher already hands tasks to compute units as they free up, so the
// metadata is an order.  Workgroup i runs on XCD i % 8 (each XCD has its own
// L2).  When Hq is a multiple of 8, XCD x owns the q-heads [x*Hq/8,
// (x+1)*Hq/8), with all their sequences and Q tiles, so the eight shares have
// the same shape and a kv-head's K/V stays within one or two XCDs; the share's
// tasks are sorted by decreasing cost (the number of KV tiles the prefill
// visits for them) so that long tasks start first and short ones fill the
// tail, and its j-th task is written at launch position 8j + x.  Otherwise
// all tasks form one list sorted the same way.  Equal costs keep increasing
// task id, which makes the order a pure function of the inputs.
//
// Four small kernels, all on the caller's stream:
//   cost     one wave per task: counts the tiles the prefill will visit
//            (mask bits or valid list entries inside the candidate range) and
//            stores the bin share*1024 + 1023 - min(cost, 1023).
//   rank     one workgroup per 1024 consecutive tasks: the bin histogram of
//            the block, and each task's rank among the block's tasks of its
//            bin with smaller id (waves take turns, in order, at a shared LDS
//            counter per bin).
//   scan     one workgroup per share: per-bin totals, an exclusive scan over
//            the share's bins in increasing order, then the start of every
//            (block, bin) pair.
//   scatter  one thread per task: its sorted position start(block, bin) +
//            rank, mapped to the launch position of its XCD share.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsa_fp8.h"
#include "bsa_internal.h"

namespace {

using bsa::candidate_end;
using bsa::kTile;

constexpr int kBuckets = 1024;        // cost buckets per share; costs above 1023 share the last
constexpr int kXcds = 8;              // XCDs of the chip: workgroup i runs on XCD i % 8
constexpr int kMaxBins = kXcds * kBuckets;
constexpr int kBlockTasks = 1024;     // tasks per rank block (and threads of the rank/scan kernels)
constexpr int kCostWaves = 4;         // tasks (waves) per workgroup of the cost kernel

struct SchedParams {
  const int32_t* cu_q;
  const int32_t* seqlens_kv;
  const uint8_t* mask;
  const int32_t* sidx;
  const int32_t* slen;
  int32_t* key;        // [N] bucket of every task
  int32_t* rank;       // [N] rank inside (block, bucket)
  int32_t* blockhist;  // [nblk, nbins] counts, then starts
  int32_t* schedule;   // [N]
  int N, nblk;
  int nbins;           // kBuckets * shares
  int heads_per_share; // Hq / 8 with shares, else Hq
  int mask_dwords;     // mask rows start on 4-byte boundaries: read them as dwords
  int Hq, mt_grid, mt, mkv, causal;
};

template <int FORM>
__global__ void __launch_bounds__(64 * kCostWaves) sched_cost_kernel(SchedParams p) {
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * kCostWaves + (threadIdx.x >> 6);
  if (task >= p.N) return;  // uniform per wave
  const int m = task % p.mt_grid;
  const int bh = task / p.mt_grid;
  const int b = bh / p.Hq;
  const int t0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - t0;
  const int lkv = p.seqlens_kv[b];
  int cost = 0;
  if (m * kTile < lq) {
    int n_end = candidate_end(lq, lkv, m, p.causal);
    const int64_t row = (int64_t)bh * p.mt + m;
    if constexpr (FORM == bsa::kFormDense) {
      cost = n_end;
    } else if constexpr (FORM == bsa::kFormMask) {
      n_end = min(n_end, p.mkv);
      const uint8_t* r = p.mask + row * p.mkv;
      if (p.mask_dwords) {
        // four mask bytes per lane; bytes at or beyond n_end are not counted
        const uint32_t* rw = reinterpret_cast<const uint32_t*>(r);
        for (int base = 0; base < n_end; base += 256) {
          const int i = base + lane * 4;
          const uint32_t w = i < n_end ? rw[i >> 2] : 0u;
#pragma unroll
          for (int k = 0; k < 4; ++k) cost += __popcll(__ballot(i + k < n_end && ((w >> (8 * k)) & 0xffu) != 0));
        }
      } else {
        for (int base = 0; base < n_end; base += 64) {
          const int i = base + lane;
          cost += __popcll(__ballot(i < n_end && r[i] != 0));
        }
      }
    } else {
      const int len = min(max(p.slen[row], 0), p.mkv);
      const int32_t* r = p.sidx + row * p.mkv;
      for (int base = 0; base < len; base += 64) {
        const int i = base + lane;
        const int e = i < len ? r[i] : -1;
        cost += __popcll(__ballot(e >= 0 && e < n_end));
      }
    }
  }
  const int share = (bh % p.Hq) / p.heads_per_share;
  if (lane == 0) p.key[task] = share * kBuckets + (kBuckets - 1 - min(cost, kBuckets - 1));
}

__global__ void __launch_bounds__(kBlockTasks) sched_rank_kernel(SchedParams p) {
  __shared__ int cnt[kMaxBins];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int task = blockIdx.x * kBlockTasks + tid;
  const bool has = task < p.N;
  const int k = has ? p.key[task] : -1;
  for (int i = tid; i < p.nbins; i += kBlockTasks) cnt[i] = 0;
  // Rank among the lanes of this wave with the same bucket and a lower lane
  // id, and whether this lane is the last of them.
  int below = 0, same = 0;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const int kj = __builtin_amdgcn_readlane(k, j);
    const bool eq = kj == k;
    below += (eq && j < lane) ? 1 : 0;
    same += eq ? 1 : 0;
  }
  const bool last = below + 1 == same;
  int r = 0;
  // Waves in order: wave w adds its lanes after waves 0..w-1.
  for (int w = 0; w < kBlockTasks / 64; ++w) {
    __syncthreads();
    if (wave == w && has) {
      r = cnt[k] + below;
      if (last) cnt[k] = r + 1;
    }
  }
  __syncthreads();
  if (has) p.rank[task] = r;
  for (int i = tid; i < p.nbins; i += kBlockTasks) p.blockhist[(int64_t)blockIdx.x * p.nbins + i] = cnt[i];
}

// One workgroup per share (a 1024-bin slice of the bins); thread t owns bin
// share*1024 + t, so every load of a histogram row is coalesced.  A share's
// tasks start at share * N/8 in sorted order (every share holds N/8 tasks), so
// the shares are scanned independently.
__global__ void __launch_bounds__(kBlockTasks) sched_scan_kernel(SchedParams p) {
  constexpr int kWaves = kBlockTasks / 64;
  constexpr int kRows = 8;  // histogram rows loaded together
  __shared__ int wsum[kWaves];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int share = (int)blockIdx.x;
  int32_t* col = p.blockhist + share * kBuckets + t;
  int tot = 0;
  for (int blk0 = 0; blk0 < p.nblk; blk0 += kRows) {
    int v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) v[r] = blk0 + r < p.nblk ? col[(int64_t)(blk0 + r) * p.nbins] : 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) tot += v[r];
  }
  // exclusive scan over the share's bins: inside the wave, then wave offsets
  int x = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += w < wave ? wsum[w] : 0;
  int run = share * (p.N / (p.nbins / kBuckets)) + before + x - tot;
  // start of every (block, bin) pair, written over the counts
  for (int blk0 = 0; blk0 < p.nblk; blk0 += kRows) {
    int v[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) v[r] = blk0 + r < p.nblk ? col[(int64_t)(blk0 + r) * p.nbins] : 0;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (blk0 + r < p.nblk) col[(int64_t)(blk0 + r) * p.nbins] = run;
      run += v[r];
    }
  }
}

__global__ void __launch_bounds__(256) sched_scatter_kernel(SchedParams p) {
  const int task = blockIdx.x * 256 + threadIdx.x;
  if (task >= p.N) return;
  const int blk = task / kBlockTasks;
  const int pos = p.blockhist[(int64_t)blk * p.nbins + p.key[task]] + p.rank[task];
  if (p.nbins == kBuckets) {
    p.schedule[pos] = task;
  } else {
    // share x = pos / (N/8) holds sorted tasks j = pos % (N/8): position 8j + x
    const int per_share = p.N / kXcds;
    const int x = pos / per_share;
    p.schedule[(pos - x * per_share) * kXcds + x] = task;
  }
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct Layout {
  int64_t key, rank, hist, total;
};

int bins_for(int num_heads_q) { return num_heads_q % kXcds == 0 ? kMaxBins : kBuckets; }

Layout workspace_layout(int64_t n, int nbins) {
  const int64_t nblk = (n + kBlockTasks - 1) / kBlockTasks;
  Layout l;
  l.key = 0;
  l.rank = align256(n * 4);
  l.hist = l.rank + align256(n * 4);
  l.total = l.hist + nblk * nbins * 4;
  return l;
}

}  // namespace

extern "C" {

long long bsa_fp8_schedule_workspace_bytes(const bsa_fp8_dims* dims) {
  bsa::Resolved r;
  if (bsa::resolve(dims, nullptr, nullptr, &r) != BSA_OK) return -1;
  if (r.tasks == 0) return 0;
  return (long long)workspace_layout(r.tasks, bins_for(r.d.num_heads_q)).total;
}

int bsa_fp8_schedule(const int32_t* cu_seqlens_q, const int32_t* seqlens_kv, const uint8_t* block_mask,
                     const bsa_fp8_dims* dims, const bsa_fp8_options* options, void* workspace,
                     int32_t* schedule, void* stream) {
  bsa_fp8_options o = {};
  if (options != nullptr) {
    o.sparse_indices = options->sparse_indices;
    o.sparse_seq_len = options->sparse_seq_len;
  }
  bsa::Resolved r;
  const int st = bsa::resolve(dims, block_mask, &o, &r);
  if (st != BSA_OK) return st;
  if (r.tasks == 0) return BSA_OK;
  if (cu_seqlens_q == nullptr || seqlens_kv == nullptr || workspace == nullptr || schedule == nullptr)
    return BSA_ERR_NULL_POINTER;

  const int nbins = bins_for(r.d.num_heads_q);
  const Layout l = workspace_layout(r.tasks, nbins);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  SchedParams p;
  p.cu_q = cu_seqlens_q;
  p.seqlens_kv = seqlens_kv;
  p.mask = block_mask;
  p.sidx = r.sidx;
  p.slen = r.slen;
  p.key = reinterpret_cast<int32_t*>(ws + l.key);
  p.rank = reinterpret_cast<int32_t*>(ws + l.rank);
  p.blockhist = reinterpret_cast<int32_t*>(ws + l.hist);
  p.schedule = schedule;
  p.N = (int)r.tasks;
  p.nblk = (int)((r.tasks + kBlockTasks - 1) / kBlockTasks);
  p.nbins = nbins;
  p.heads_per_share = nbins == kMaxBins ? r.d.num_heads_q / kXcds : r.d.num_heads_q;
  p.mask_dwords = block_mask != nullptr && (r.d.mask_tiles_kv & 3) == 0 &&
                  (reinterpret_cast<uintptr_t>(block_mask) & 3) == 0;
  p.Hq = r.d.num_heads_q;
  p.mt_grid = r.mt_grid;
  p.mt = r.d.mask_tiles_q;
  p.mkv = r.d.mask_tiles_kv;
  p.causal = r.d.causal;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 cost_grid((unsigned)((r.tasks + kCostWaves - 1) / kCostWaves));
  if (r.form == bsa::kFormList)
    hipLaunchKernelGGL(sched_cost_kernel<bsa::kFormList>, cost_grid, dim3(64 * kCostWaves), 0, s, p);
  else if (r.form == bsa::kFormMask)
    hipLaunchKernelGGL(sched_cost_kernel<bsa::kFormMask>, cost_grid, dim3(64 * kCostWaves), 0, s, p);
  else
    hipLaunchKernelGGL(sched_cost_kernel<bsa::kFormDense>, cost_grid, dim3(64 * kCostWaves), 0, s, p);
  hipLaunchKernelGGL(sched_rank_kernel, dim3((unsigned)p.nblk), dim3(kBlockTasks), 0, s, p);
  hipLaunchKernelGGL(sched_scan_kernel, dim3((unsigned)(nbins / kBuckets)), dim3(kBlockTasks), 0, s, p);
  hipLaunchKernelGGL(sched_scatter_kernel, dim3((unsigned)((r.tasks + 255) / 256)), dim3(256), 0, s, p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_LAUNCH;
  return BSA_OK;
}

}  // extern "C"
