// FP8 sparse decode over a paged cache of 656-byte token rows, gfx950.
//
// The workload of the FlashMLA FP8 sparse decoding article: multi-query
// attention (every query head reads the same single KV head) with 576-dim keys
// (512 E4M3 values in four 1x128 tiles with one float32 descale each, then 64
// bfloat16 values) and 512-dim values (the first 512 key dimensions); each
// query token attends to its own list of top-k token positions.  The article's
// kernel dequantises K/V to bfloat16 and runs both products on bfloat16 matrix
// units; the same split holds here.
//
// One workgroup (4 waves) per (sequence b, query token s, group of 64 heads);
// the top-k list is walked 32 tokens at a time:
//   A. gather + dequantise: thread t takes token t/8 of the block and one
//      eighth of its row (64 E4M3 codes, their descale, 8 bfloat16 values),
//      converts code * descale to bfloat16 (round to nearest even) and writes
//      a row-major bfloat16 K tile [32 tokens][576] to LDS.  The row bytes
//      come from a per-wave LDS staging area that direct-to-LDS loads filled
//      during the previous block; the row loads of the next block, the page
//      lookups of the block after it and the index loads of the one after
//      that are issued here, so a block's memory traffic is in flight during
//      the blocks before it is used and holds no registers meanwhile.
//   B. S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: wave w owns heads
//      16w..16w+15 with Q in registers.  K rows are read in a permuted order
//      so that each lane ends up holding 8 consecutive tokens of one head,
//      which is the layout of the P operand below.  Online softmax in the log2
//      domain (running max and sum per head); P is rounded to bfloat16 into an
//      LDS buffer [64 heads][32 tokens], with each head's rescale factor.
//   C. O^T += V^T . P^T: wave w owns output dims 128w..128w+127 for all 64
//      heads, so each V value is read from LDS once per workgroup.  V^T comes
//      straight from the row-major K tile through the transposing read
//      ds_read_b64_tr_b16.
// Epilogue: O = O_acc / l per head, bfloat16; LSE = ln sum exp(score).  A
// query with no valid index gets O = 0 and LSE = -FLT_MAX.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

#include "bsa_fp8.h"
#include "bsa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 64;          // heads per workgroup
constexpr int kBlock = 32;          // tokens per iteration
constexpr int kDimK = 576;
constexpr int kDimV = 512;
constexpr int kRowBytes = 656;
constexpr int kKStride = kDimK * 2 + 16;   // bytes per LDS K row (padded)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegFltMax = -3.402823466e+38f;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

struct DecodeParams {
  const uint16_t* q;          // bf16 [B, s_q, h_q, 576]
  const uint8_t* kv;          // [num_pages, page_size, 656]
  const int32_t* indices;     // [B, s_q, topk]
  const int32_t* block_table; // [B, max_pages]
  const int32_t* seqlens_kv;  // [B]
  uint16_t* out;              // bf16 [B, s_q, h_q, 512]
  float* lse;                 // [B, h_q, s_q] or nullptr
  int B, s_q, h_q, topk, page_size, page_shift, max_pages;
  float score_scale;          // softmax_scale * log2(e)
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

__device__ __forceinline__ v4f mfma_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                  0, 0);
}

// Direct-to-LDS loads (16 and 4 bytes per lane; a wave writes 64 consecutive
// elements at the wave-uniform LDS address lds_addr), issued through asm so
// that the compiler does not make later LDS reads and barriers wait for them;
// they are waited for explicitly (s_waitcnt vmcnt) before their data is read.
// M0 is set here and used by nothing else in this kernel.
__device__ __forceinline__ void dma_lds16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_addr) : "memory");
}
// Workgroup barrier that waits for this wave's LDS operations only; loads from
// global memory stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Per-wave staging of one thread's share of a token row: slots 0..3 hold its
// 64 codes (16 bytes per lane each), slot 4 its 8 bfloat16 values, then the
// descale (4 bytes per lane).
constexpr int kStageSlot = 64 * 16;
constexpr int kStageWave = 5 * kStageSlot + 64 * 4;

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bsa_fp8_decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBlock * kKStride];        // 37,376 B
  __shared__ __attribute__((aligned(16))) uint16_t p_lds[kHeads * kBlock];         // 4 KB
  __shared__ float alpha_lds[kHeads];
  __shared__ float l_lds[kHeads];
  __shared__ float m_lds[kHeads];
  __shared__ __attribute__((aligned(16))) uint8_t valid_lds[kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t stage_lds[4 * kStageWave];   // 21,504 B

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4;       // lane group
  const int c16 = lane & 15;     // column within a 16x16 block

  const int groups = p.h_q / kHeads;
  const int hg = blockIdx.x % groups;
  const int bs = blockIdx.x / groups;  // b * s_q + s
  const int b = bs / p.s_q;
  const int s = bs - b * p.s_q;
  const int h0 = hg * kHeads;
  const int lkv = p.seqlens_kv[b];
  const int32_t* idx_row = p.indices + (int64_t)bs * p.topk;
  const int32_t* bt = p.block_table + (int64_t)b * p.max_pages;

  // ---- Q of this wave's 16 heads (B operand of S^T = K.Q^T) -----------------
  // lane: head 16w + c16, dims 32*ks + 8*G .. +7
  v4i qreg[18];
  {
    const uint16_t* qp = p.q + ((int64_t)bs * p.h_q + h0 + wave * 16 + c16) * kDimK + 8 * G;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const v4i*>(qp + 32 * ks);
  }

  v4f oacc[8][4];  // [dim block][head block]: dims 128w + 16*db + 4G .. +3, head 16*hb + c16
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) oacc[db][hb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;  // per head (column c16 of this wave), log2 domain
  float l_run = 0.0f;       // this lane's share of the row sum

  const int nblocks = lkv > 0 ? (p.topk + kBlock - 1) / kBlock : 0;

  // ---- index -> row pipeline for this thread's token (token tid/8 of a block)
  const int tok = tid >> 3;
  const int part = tid & 7;
  // a row that is always readable: position 0 of the sequence
  const int fallback_row = lkv > 0 ? bt[0] * p.page_size : 0;
  auto load_index = [&](int n) -> int {
    const int k = n * kBlock + tok;
    return (n < nblocks && k < p.topk) ? idx_row[k] : -1;
  };
  // row id (page * page_size + slot), or -1 for an entry that selects nothing
  auto lookup_row = [&](int idx) -> int {
    const bool ok = idx >= 0 && idx < lkv;
    const int pg = bt[ok ? (idx >> p.page_shift) : 0];
    return ok ? pg * p.page_size + (idx & (p.page_size - 1)) : -1;
  };
  uint8_t* stage = stage_lds + wave * kStageWave;
  const uint32_t stage_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)stage);
  auto stage_row = [&](int row) {
    const uint8_t* r = p.kv + (int64_t)(row >= 0 ? row : fallback_row) * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_lds16(r + part * 64 + 16 * i, stage_addr + i * kStageSlot);
    dma_lds16(r + kDimV + 16 + 16 * part, stage_addr + 4 * kStageSlot);
    dma_lds4(r + kDimV + 4 * (part >> 1), stage_addr + 5 * kStageSlot);
  };

  int row_cur = -1;   // row of block n (being dequantised)
  int row_next = -1;  // row of block n+1
  int idx_next2 = -1; // index of block n+2
  if (nblocks > 0) {
    row_cur = lookup_row(load_index(0));
    stage_row(row_cur);
    row_next = lookup_row(load_index(1));
    idx_next2 = load_index(2);
  }

  for (int n = 0; n < nblocks; ++n) {
    // ---- A: dequantise block n into the K tile ------------------------------
    wait_all_loads();  // this block's staged rows and the next lookups have arrived
    lds_barrier();     // the previous block's K tile and P buffer are no longer read
    {
      uint8_t* dst = k_lds + tok * kKStride;
      const float scale = *reinterpret_cast<const float*>(stage + 5 * kStageSlot + 4 * lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i codes = *reinterpret_cast<const v4i*>(stage + i * kStageSlot + 16 * lane);
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c = (uint32_t)codes[j];
          const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
          const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
          w[2 * j] = pack_bf16(lo[0] * scale, lo[1] * scale);
          w[2 * j + 1] = pack_bf16(hi[0] * scale, hi[1] * scale);
        }
        *reinterpret_cast<v4i*>(dst + 2 * (part * 64 + 16 * i)) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        *reinterpret_cast<v4i*>(dst + 2 * (part * 64 + 16 * i + 8)) =
            v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
      }
      *reinterpret_cast<v4i*>(dst + 2 * (kDimV + 8 * part)) =
          *reinterpret_cast<const v4i*>(stage + 4 * kStageSlot + 16 * lane);
      if (part == 0) valid_lds[tok] = row_cur >= 0 ? 1 : 0;
    }
    // next loads: rows of block n+1 (into the staging area, once this wave's
    // reads of it are complete), page lookups of block n+2, indices of n+3
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    row_cur = row_next;
    if (n + 1 < nblocks) stage_row(row_cur);
    row_next = lookup_row(idx_next2);
    idx_next2 = load_index(n + 3);
    lds_barrier();  // K tile ready

    // ---- B: S^T = K . Q^T for heads 16w..16w+15 --------------------------------
    // block c, accumulator row m -> token 8*(m/4) + 4c + m%4; lane (G, c16) then
    // holds tokens 8G .. 8G+7 of head c16 in s[0][0..3], s[1][0..3].
    v4f sacc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
    {
      const int tok0 = 8 * (c16 >> 2) + (c16 & 3);
      const uint8_t* a0 = k_lds + tok0 * kKStride + 2 * 8 * G;
      const uint8_t* a1 = a0 + 4 * kKStride;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        const v4i ka = *reinterpret_cast<const v4i*>(a0 + 64 * ks);
        const v4i kb = *reinterpret_cast<const v4i*>(a1 + 64 * ks);
        sacc[0] = mfma_bf16(ka, qreg[ks], sacc[0]);
        sacc[1] = mfma_bf16(kb, qreg[ks], sacc[1]);
      }
    }
    // online softmax for head c16 over tokens 8G..8G+7
    {
      const uint64_t vbits = *reinterpret_cast<const uint64_t*>(valid_lds + 8 * G);
      float x[8];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (vbits >> (8 * (4 * c + r))) & 0xff;
          x[4 * c + r] = ok ? sacc[c][r] * p.score_scale : -INFINITY;
        }
      float bmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run, bmax);
      const float m_safe = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_safe);  // 0 while nothing was seen
      float e[8];
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = __builtin_amdgcn_exp2f(x[i] - m_safe);
        sum += e[i];
      }
      l_run = l_run * alpha + sum;
      m_run = m_new;
      const v4i pk = v4i{(int)pack_bf16(e[0], e[1]), (int)pack_bf16(e[2], e[3]), (int)pack_bf16(e[4], e[5]),
                         (int)pack_bf16(e[6], e[7])};
      *reinterpret_cast<v4i*>(p_lds + (wave * 16 + c16) * kBlock + 8 * G) = pk;
      if (G == 0) alpha_lds[wave * 16 + c16] = alpha;
    }
    lds_barrier();  // P and rescale factors ready

    // ---- C: O^T += V^T . P^T for dims 128w.., all 64 heads -----------------------
    {
      float al[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) al[hb] = alpha_lds[16 * hb + c16];
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) oacc[db][hb] *= al[hb];
      v4i pb[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pb[hb] = *reinterpret_cast<const v4i*>(p_lds + (16 * hb + c16) * kBlock + 8 * G);
      // transposing reads: source lane (G, j) addresses token 8G + j/4 (+4),
      // dims d0 + 4*(j%4); result lane (G, i) then holds dim d0 + i of tokens
      // 8G .. 8G+7
      const uint8_t* vbase = k_lds + (8 * G + (c16 >> 2)) * kKStride + 2 * (128 * wave + 4 * (c16 & 3));
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase + 2 * 16 * db));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vbase + 4 * kKStride + 2 * 16 * db));
        const v2i l2 = __builtin_bit_cast(v2i, lo);
        const v2i h2 = __builtin_bit_cast(v2i, hi);
        const v4i va = v4i{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) oacc[db][hb] = mfma_bf16(va, pb[hb], oacc[db][hb]);
      }
    }
  }

  // ---- epilogue ----------------------------------------------------------------
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  wait_all_loads();  // no load is left in flight when the workgroup ends
  __syncthreads();
  if (G == 0) {
    l_lds[wave * 16 + c16] = l_tot;
    m_lds[wave * 16 + c16] = m_run;
  }
  __syncthreads();
  if (p.lse != nullptr && G == 0) {
    const bool empty = !(l_tot > 0.0f);
    p.lse[((int64_t)b * p.h_q + h0 + wave * 16 + c16) * p.s_q + s] =
        empty ? kNegFltMax : (m_run + log2f(l_tot)) * kLn2;
  }
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float l = l_lds[16 * hb + c16];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* op = p.out + ((int64_t)bs * p.h_q + h0 + 16 * hb + c16) * kDimV + 128 * wave + 4 * G;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4f o = oacc[db][hb] * inv;
      *reinterpret_cast<v2i*>(op + 16 * db) = v2i{(int)pack_bf16(o[0], o[1]), (int)pack_bf16(o[2], o[3])};
    }
  }
}

}  // namespace

extern "C" {

int bsa_fp8_sparse_decode(const void* q, const void* kv_cache, const int32_t* indices,
                          const int32_t* block_table, const int32_t* seqlens_kv,
                          const bsa_fp8_decode_dims* dims, void* out, float* lse, void* stream) {
  if (dims == nullptr) return BSA_ERR_NULL_POINTER;
  const bsa_fp8_decode_dims d = *dims;
  if (d.batch < 0 || d.s_q < 0 || d.num_heads_q <= 0 || d.topk <= 0 || d.num_pages < 0 ||
      d.max_pages_per_seq < 0)
    return BSA_ERR_SIZE;
  if (d.num_heads_q % kHeads != 0) return BSA_ERR_GQA;
  if (d.page_size != 32 && d.page_size != 64) return BSA_ERR_PAGE_SIZE;
  if (!bsa::finite_float(d.softmax_scale)) return BSA_ERR_SOFTMAX_SCALE;
  const int64_t grid = (int64_t)d.batch * d.s_q * (d.num_heads_q / kHeads);
  if (grid > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;
  if ((int64_t)d.num_pages * d.page_size > 0x7fffffffLL) return BSA_ERR_TOO_LARGE;  // 32-bit row ids
  if (grid == 0) return BSA_OK;
  if (q == nullptr || kv_cache == nullptr || indices == nullptr || block_table == nullptr ||
      seqlens_kv == nullptr || out == nullptr)
    return BSA_ERR_NULL_POINTER;

  DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.indices = indices;
  p.block_table = block_table;
  p.seqlens_kv = seqlens_kv;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.B = d.batch;
  p.s_q = d.s_q;
  p.h_q = d.num_heads_q;
  p.topk = d.topk;
  p.page_size = d.page_size;
  p.page_shift = d.page_size == 64 ? 6 : 5;
  p.max_pages = d.max_pages_per_seq;
  p.score_scale = d.softmax_scale * kLog2e;
  hipLaunchKernelGGL(bsa_fp8_decode_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_LAUNCH;
  return BSA_OK;
}

}  // extern "C"
