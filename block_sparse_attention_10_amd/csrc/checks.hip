// Checks of the data-dependent inputs, run before a call's kernels when the
// descriptor sets MSA_FLAG_DEBUG_CHECKS.
//
// The fast path trusts ctx_lens, the block table, selections handed to the
// page-table build and page tables handed to the attention for its results
// (the kernels clamp the block ids they dereference, so a bad entry reads
// or writes the wrong place inside the caller's buffers).  In debug mode
// one workgroup reads those inputs, records the first violation of each
// kind, and the host reads the record back (the call synchronises its
// stream) before anything else is launched, so a bad input is reported and
// never used.
//
// What each kind checks (B requests, T rows each, MAXB table columns, NB
// physical blocks, block size 128, 8 pages per block):
//   context   T <= ctx_lens[b] <= MAXB * 128;
//   table     0 <= block_table[b][c] < NB for the blocks a call reads: every
//             block of the context (c <= (L - 1) / 128), or only the blocks
//             of the T newest tokens (the write path);
//   selection selected[r][k] is -1 or a logical block c < MAXB whose table
//             entry is a physical block;
//   pages     each group of 8 entries of a page-table row is all -1 or the
//             pages 8 phys .. 8 phys + 7 of one physical block phys < NB,
//             the first group is real and no real group follows a -1 group
//             (the attention reads the groups in order and takes the last
//             one as the row's local block).
#include "msa_internal.h"

#include <limits.h>

#include <mutex>

namespace msa {
namespace {

constexpr int kThreads = 1024;
constexpr int kKinds = 4;  // context, table, selection, pages

// Per device: for each kind the first violation as (flat index * 4 +
// reason), or -1, then the offending value and a second value.
__device__ long long g_check_record[3 * kKinds];

__device__ __forceinline__ void note_first(unsigned long long* slot, long long index,
                                           int reason) {
  atomicMin(slot, (unsigned long long)(index * 4 + reason));
}

__device__ __forceinline__ bool context_ok(int L, int T, int MAXB) {
  return L >= T && (long long)L <= (long long)MAXB * 128;
}

__global__ __launch_bounds__(kThreads) void input_check_kernel(CheckInputs a) {
  __shared__ unsigned long long first[kKinds];
  const int tid = threadIdx.x;
  if (tid < kKinds) first[tid] = ULLONG_MAX;
  __syncthreads();
  const long long R = (long long)a.B * a.T;

  if (a.ctx_lens) {
    for (int b = tid; b < a.B; b += kThreads)
      if (!context_ok(a.ctx_lens[b], a.T, a.MAXB)) note_first(&first[0], b, 0);
  }
  if (a.block_table && a.ctx_lens) {
    const long long n = (long long)a.B * a.MAXB;
    for (long long i = tid; i < n; i += kThreads) {
      const int b = (int)(i / a.MAXB);
      const int c = (int)(i - (long long)b * a.MAXB);
      const int L = a.ctx_lens[b];
      if (!context_ok(L, a.T, a.MAXB)) continue;  // reported as a context
      const int lo = a.new_tokens_only ? (L - a.T) / 128 : 0;
      if (c < lo || c > (L - 1) / 128) continue;
      const int v = a.block_table[i];
      if (v < 0 || v >= a.NB) note_first(&first[1], i, 0);
    }
  }
  if (a.selected && a.block_table) {
    const long long n = R * a.topk;
    for (long long i = tid; i < n; i += kThreads) {
      const int b = (int)(i / a.topk / a.T);
      const int c = a.selected[i];
      if (c == -1) continue;
      if (c < 0 || c >= a.MAXB) {
        note_first(&first[2], i, 1);
        continue;
      }
      const int v = a.block_table[(long long)b * a.MAXB + c];
      if (v < 0 || v >= a.NB) note_first(&first[2], i, 2);
    }
  }
  if (a.page_table) {
    const int groups = a.topk;
    const long long n = R * groups;
    for (long long i = tid; i < n; i += kThreads) {
      const long long r = i / groups;
      const int k = (int)(i - r * groups);
      const int32_t* g = a.page_table + r * (8LL * groups) + 8 * k;
      const int p0 = g[0];
      if (p0 == -1) {
        if (k == 0) {  // a row of padding only
          bool any = false;
          for (int kk = 1; kk < groups; ++kk) any = any || g[8 * kk] != -1;
          if (!any) note_first(&first[3], i, 0);
        }
        for (int j = 1; j < 8; ++j)
          if (g[j] != -1) {
            note_first(&first[3], i, 2);
            break;
          }
        continue;
      }
      if (p0 < 0 || (p0 & 7) != 0 || (p0 >> 3) >= a.NB) {
        note_first(&first[3], i, 1);
        continue;
      }
      bool run = true;
      for (int j = 1; j < 8; ++j) run = run && g[j] == p0 + j;
      if (!run) {
        note_first(&first[3], i, 2);
        continue;
      }
      if (k > 0 && g[-8] == -1) note_first(&first[3], i, 3);
    }
  }
  __syncthreads();

  if (tid < kKinds) {
    const unsigned long long f = first[tid];
    long long key = -1, v0 = 0, v1 = 0;
    if (f != ULLONG_MAX) {
      key = (long long)f;
      const long long i = key >> 2;
      if (tid == 0) {
        v0 = a.ctx_lens[i];
      } else if (tid == 1) {
        v0 = a.block_table[i];
      } else if (tid == 2) {
        v0 = a.selected[i];
        if ((key & 3) == 2)
          v1 = a.block_table[(i / a.topk / a.T) * a.MAXB + v0];
      } else {
        const long long r = i / a.topk, k = i - r * a.topk;
        v0 = a.page_table[r * 8 * a.topk + 8 * k];
      }
    }
    g_check_record[3 * tid] = key;
    g_check_record[3 * tid + 1] = v0;
    g_check_record[3 * tid + 2] = v1;
  }
}

std::mutex g_check_mutex;  // the record is one per device

std::string describe(const CheckInputs& a, const long long* rec) {
  std::string s;
  for (int k = 0; k < kKinds && s.empty(); ++k) {
    const long long key = rec[3 * k];
    if (key < 0) continue;
    const long long i = key >> 2, v0 = rec[3 * k + 1], v1 = rec[3 * k + 2];
    const int reason = (int)(key & 3);
    const std::string T = std::to_string(a.T), MAXB = std::to_string(a.MAXB),
                      NB = std::to_string(a.NB);
    if (k == 0) {
      s = "ctx_lens[" + std::to_string(i) + "] = " + std::to_string(v0) + ": needs " + T +
          " <= L <= max_blocks_per_seq * 128 = " + std::to_string((long long)a.MAXB * 128);
    } else if (k == 1) {
      s = "block_table[" + std::to_string(i / a.MAXB) + "][" + std::to_string(i % a.MAXB) +
          "] = " + std::to_string(v0) + ": a block of the context outside [0, " + NB + ")";
    } else if (k == 2) {
      const std::string at =
          "selected[" + std::to_string(i / a.topk) + "][" + std::to_string(i % a.topk) + "] = ";
      s = reason == 1 ? at + std::to_string(v0) + ": neither -1 nor a block id in [0, " + MAXB +
                            ")"
                      : at + std::to_string(v0) + " maps to block_table entry " +
                            std::to_string(v1) + " outside [0, " + NB + ")";
    } else {
      const std::string at = "page_table[" + std::to_string(i / a.topk) + "][" +
                             std::to_string(8 * (i % a.topk)) + "..+7] (first " +
                             std::to_string(v0) + "): ";
      if (reason == 0)
        s = at + "the row has no block (its local block comes last)";
      else if (reason == 1)
        s = at + "not the pages 8 phys .. 8 phys + 7 of a block phys in [0, " + NB + ")";
      else if (reason == 2)
        s = at + "the 8 entries are neither all -1 nor consecutive pages of one block";
      else
        s = at + "a block follows -1 padding";
    }
  }
  return s;
}

}  // namespace

hipError_t run_input_checks(const CheckInputs& a, hipStream_t s, std::string* failure) {
  std::lock_guard<std::mutex> lock(g_check_mutex);
  hipLaunchKernelGGL(input_check_kernel, dim3(1), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the kernel wrote the record of the device that runs `s`; the symbol
  // copy resolves the record of the current device, so that device is made
  // current for it
  int dev = 0, cur = 0;
  if ((e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
  if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
  long long rec[3 * kKinds];
  e = hipMemcpyFromSymbolAsync(rec, HIP_SYMBOL(g_check_record), sizeof(rec), 0,
                               hipMemcpyDeviceToHost, s);
  if (dev != cur) {
    const hipError_t back = hipSetDevice(cur);
    if (e == hipSuccess) e = back;
  }
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *failure = describe(a, rec);
  return hipSuccess;
}

}  // namespace msa
