// Top-k block selection: one workgroup selects for every row of a request.
//
// aisoku.org MiniMax-M3.1-Flash article, section "MSAの仕組み", and the
// agentlenshq page, section "MSA 実行プロセス" step 2 (local_blocks = 1): each
// row keeps its local block (the one holding the query token) plus the best
// of the other causal blocks, topk blocks in all.  Ties go to the lower block
// id; the kept ids are emitted ascending.  news.ainew.jp MI355X article,
// section 2: one workgroup per request covers all draft positions.
//
// Design: a row's candidates are spread over 1, 2 or 4 waves (4 / T when
// T < 4).  Every lane streams its candidates in ascending id order into a
// register-resident sorted list of the topk - 1 best 64-bit keys (orderable
// score << 32 | ~id, so a larger key is a better block and equal scores
// favour the lower id).  Each wave then pops its topk - 1 best keys by
// repeated wave maxima (DPP reductions, no LDS traffic), the waves of a row
// meet in LDS, and one wave ranks the union (at most 60 finalists, one per
// lane), sorts the winners by id and writes the row's selection and page
// table.
#pragma once

#include "msa_device.h"

namespace msa {

constexpr int kMaxTopk = 16;
constexpr int kList = kMaxTopk - 1;  // per-lane list length (non-local picks)
constexpr int kBatch = 16;           // score loads in flight per lane

// Monotone map fp32 -> uint32 for a total order; NaN ranks as -inf and -0
// as +0.
__device__ __forceinline__ uint32_t orderable(float s) {
  if (s != s) s = -INFINITY;
  if (s == 0.f) s = 0.f;
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, int c) {
  return ((uint64_t)orderable(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
}

__device__ __forceinline__ int key_id(uint64_t k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu));
}

// LDS a selecting workgroup needs.
struct SelectLds {
  uint64_t finalists[4 * kList];  // wave w's picks at [w * K1, w * K1 + K1)
  int32_t row_sel[4][kMaxTopk];
};

// Selection (and, when page_table is given, the page table) for every row of
// request b.  Called by all 256 threads of a 4-wave workgroup; contains
// workgroup barriers.
__device__ __forceinline__ void select_request(int b, const float* __restrict__ scores,
                                            const int32_t* __restrict__ ctx_lens,
                                            const int32_t* __restrict__ block_table,
                                            int32_t* __restrict__ selected,
                                            int32_t* __restrict__ n_selected,
                                            int32_t* __restrict__ page_table, int T, int MAXB,
                                            int topk, SelectLds& sh) {
  uint64_t* finalists = sh.finalists;
  auto& row_sel = sh.row_sel;
  const int lane = lane_id();
  const int wave = wave_id();
  const int L = ctx_lens[b];
  const int parts = T >= 4 ? 1 : (T == 1 ? 4 : (T == 2 ? 2 : 1));
  const int rows_per_pass = 4 / parts;
  const int K1 = topk - 1;

  for (int t0 = 0; t0 < T; t0 += rows_per_pass) {
    const int t = t0 + wave / parts;
    const int part = wave % parts;
    const bool active = t < T;
    const int pos = L - T + t;
    const int local = pos >> 7;
    const bool take_all = local + 1 <= topk;
    const int r = b * T + t;

    if (active && !take_all && K1 > 0) {
      const float* srow = scores + (size_t)r * MAXB;
      uint64_t list[kList];
#pragma unroll
      for (int j = 0; j < kList; ++j) list[j] = 0;  // 0 ranks below every real key
      // batches of kBatch independent score loads per lane, then insertion
      const int stride = parts * kWave;
      for (int c0 = part * kWave + lane; c0 < local; c0 += kBatch * stride) {
        float sv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * stride;
          sv[u] = c < local ? srow[c] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * stride;
          if (c >= local) break;
          uint64_t x = make_key(sv[u], c);
          if (x > list[kList - 1]) {
#pragma unroll
            for (int j = 0; j < kList; ++j) {
              const uint64_t y = list[j];
              const bool gt = x > y;
              list[j] = gt ? x : y;
              x = gt ? y : x;
            }
          }
        }
      }
      for (int k = 0; k < K1; ++k) {
        const uint64_t best = wave_max_u64(list[0]);
        if (lane == 0) finalists[wave * K1 + k] = best;
        if (best != 0 && list[0] == best) {
#pragma unroll
          for (int j = 0; j < kList - 1; ++j) list[j] = list[j + 1];
          list[kList - 1] = 0;
        }
      }
    }
    __syncthreads();

    if (active && part == 0) {
      int n = 0;
      if (take_all) {
        n = local + 1;
        for (int k = lane; k < n; k += kWave) row_sel[wave][k] = k;
      } else if (K1 == 0) {
        if (lane == 0) row_sel[wave][0] = local;
        n = 1;
      } else {
        // rank the union of this row's per-wave lists; keys are unique
        // the row's waves are wave .. wave + parts - 1: their picks are contiguous
        const int m = parts * K1;
        const uint64_t* fin = finalists + wave * K1;
        const uint64_t mine = lane < m ? fin[lane] : 0;
        int rank = 0;
        for (int e = 0; e < m; ++e) rank += fin[e] > mine ? 1 : 0;
        const bool win = lane < m && rank < K1 && mine != 0;
        const int id = key_id(mine);
        // position among the winners by ascending id
        __builtin_amdgcn_wave_barrier();
        if (win) row_sel[wave][rank] = id;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int posn = 0;
        if (win)
          for (int e = 0; e < K1; ++e) posn += row_sel[wave][e] < id ? 1 : 0;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (win) row_sel[wave][posn] = id;
        if (lane == 0) row_sel[wave][K1] = local;
        n = topk;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (selected)
        for (int k = lane; k < topk; k += kWave)
          selected[(size_t)r * topk + k] = k < n ? row_sel[wave][k] : -1;
      if (lane == 0 && n_selected) n_selected[r] = n;
      if (page_table) {
        const int pt = topk * 8;
        for (int e = lane; e < pt; e += kWave) {
          const int k = e >> 3;
          int v = -1;
          if (k < n) v = block_table[(size_t)b * MAXB + row_sel[wave][k]] * 8 + (e & 7);
          page_table[(size_t)r * pt + e] = v;
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace msa
