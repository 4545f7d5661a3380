// Counter driver for rocprofv3 --pmc runs.
//
// Launches the library's entry points on the shapes, context lengths and
// block table of a workload (a spec file written by synth.write_spec), with
// no Python or torch in the process, or a plain device copy of known size
// for calibrating the memory counters:
//
//   msa_counters scan   <spec> <launches>   msa_index_score x launches
//   msa_counters decode <spec> <launches>   msa_decode x launches
//   msa_counters decode <spec> <launches> flush
//                                           each msa_decode after a 1 GiB copy
//                                           (caches and TLBs hold other data)
//   msa_counters copy   <MiB>  <launches>   16-byte copy kernel x launches
//
// Index keys and queries hold hashed small integers in [-8, 8] (so the
// selections differ from row to row, as with real data); K / V pool contents
// are constants (1.0 in every format): the bytes a kernel moves do not
// depend on them.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <fstream>
#include <string>
#include <vector>

#include "msa.h"

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void copy16(const u32x4* __restrict__ in, u32x4* __restrict__ out, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = in[i];
}

__global__ void fill_u16(uint16_t* p, size_t n, uint16_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Integers in [-8, 8] from a 32-bit hash of the element index, stored as
// bf16 (BYTES == 2) or e4m3 codes (BYTES == 1); both are exact.  The hash
// is Chris Wellons' published "lowbias32" integer mixer (hash-prospector
// project: xorshift 16, multiply 0x7feb352d, xorshift 15, multiply
// 0x846ca68b, xorshift 16).
__device__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}
__constant__ uint8_t kE4m3Int[17] = {0xD0, 0xCE, 0xCC, 0xCA, 0xC8, 0xC4, 0xC0, 0xB8, 0x00,
                                     0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50};
template <int BYTES>
__global__ void fill_small_ints(void* p, size_t n, uint32_t salt) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const int v = (int)(hash32((uint32_t)i ^ salt) % 17u) - 8;
    if (BYTES == 2) {
      const float f = (float)v;
      ((uint16_t*)p)[i] = (uint16_t)(__float_as_uint(f) >> 16);
    } else {
      ((uint8_t*)p)[i] = kE4m3Int[v + 8];
    }
  }
}

__global__ void fill_hash_bytes(uint8_t* p, size_t n, uint32_t salt) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = (uint8_t)hash32((uint32_t)i ^ salt);
}

__global__ void fill_f32(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

static void* dalloc(size_t bytes) {
  void* p = nullptr;
  CHECK(hipMalloc(&p, bytes < 256 ? 256 : bytes));
  return p;
}

static int dtype_code(const std::string& s) {
  if (s == "bf16") return MSA_DTYPE_BF16;
  if (s == "fp8") return MSA_DTYPE_FP8_E4M3;
  return MSA_DTYPE_NVFP4;
}

int main(int argc, char** argv) {
  const bool flush = argc == 5 && std::string(argv[4]) == "flush";
  if (argc != 4 && !flush) {
    fprintf(stderr,
            "usage: %s scan|decode <spec> <launches> [flush] | copy <MiB> <launches>\n",
            argv[0]);
    return 2;
  }
  const std::string mode = argv[1];
  const int launches = atoi(argv[3]);
  if (mode == "copy") {
    const size_t bytes = (size_t)atol(argv[2]) << 20;
    void* a = dalloc(bytes);
    void* b = dalloc(bytes);
    CHECK(hipMemset(a, 1, bytes));
    for (int i = 0; i < launches; ++i)
      hipLaunchKernelGGL(copy16, dim3(4096), dim3(256), 0, 0, (const u32x4*)a, (u32x4*)b,
                         bytes / 16);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    printf("copy bytes_per_launch %zu launches %d\n", bytes, launches);
    return 0;
  }

  std::ifstream f(argv[2]);
  int B, T, Hq, Hkv, Hidx, MAXB, NB, topk;
  std::string kv, idx;
  if (!(f >> B >> T >> Hq >> Hkv >> Hidx >> MAXB >> NB >> kv >> idx >> topk)) {
    fprintf(stderr, "bad spec header\n");
    return 2;
  }
  std::vector<int32_t> ctx(B), bt((size_t)B * MAXB);
  for (auto& x : ctx) f >> x;
  for (auto& x : bt) f >> x;
  if (!f) {
    fprintf(stderr, "bad spec body\n");
    return 2;
  }
  const size_t R = (size_t)B * T;
  const int kvc = dtype_code(kv), idc = dtype_code(idx);
  // index-key bytes per element: bf16 2, fp8 1 (4-bit: half a byte, below)
  const size_t ie = idc == MSA_DTYPE_BF16 ? 2 : 1;
  const size_t rows = (size_t)NB * Hkv * 128;
  const size_t kv_row = kvc == MSA_DTYPE_BF16 ? 256 : (kvc == MSA_DTYPE_FP8_E4M3 ? 128 : 64);

  msa_problem p;
  memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.batch = B; p.decode_query_len = T; p.num_q_heads = Hq; p.num_kv_heads = Hkv;
  p.num_idx_heads = Hidx; p.head_dim = 128; p.idx_dim = 64; p.block_size = 128;
  p.page_size = 16; p.topk = topk; p.local_blocks = 1; p.max_blocks_per_seq = MAXB;
  p.num_phys_blocks = NB; p.kv_dtype = kvc; p.idx_k_dtype = idc;

  msa_tensors t;
  memset(&t, 0, sizeof(t));
  int32_t* d_ctx = (int32_t*)dalloc(B * 4);
  int32_t* d_bt = (int32_t*)dalloc(bt.size() * 4);
  CHECK(hipMemcpy(d_ctx, ctx.data(), B * 4, hipMemcpyHostToDevice));
  CHECK(hipMemcpy(d_bt, bt.data(), bt.size() * 4, hipMemcpyHostToDevice));
  t.ctx_lens = d_ctx;
  t.block_table = d_bt;
  uint16_t* iq = (uint16_t*)dalloc(R * Hidx * 64 * 2);
  hipLaunchKernelGGL(fill_small_ints<2>, dim3(256), dim3(256), 0, 0, iq, R * Hidx * 64, 17u);
  t.idx_q = iq;
  const size_t ik_elems = (size_t)NB * Hidx * 128 * 64;
  void* ik;
  if (idc == MSA_DTYPE_NVFP4) {
    // random E2M1 code pairs, every scale 2.0
    ik = dalloc(ik_elems / 2);
    hipLaunchKernelGGL(fill_hash_bytes, dim3(4096), dim3(256), 0, 0, (uint8_t*)ik, ik_elems / 2,
                       91u);
    void* iks = dalloc(ik_elems / 16);
    CHECK(hipMemset(iks, 0x40, ik_elems / 16));
    t.idx_k_scale = iks;
  } else {
    ik = dalloc(ik_elems * ie);
    if (ie == 2)
      hipLaunchKernelGGL(fill_small_ints<2>, dim3(4096), dim3(256), 0, 0, ik, ik_elems, 91u);
    else
      hipLaunchKernelGGL(fill_small_ints<1>, dim3(4096), dim3(256), 0, 0, ik, ik_elems, 91u);
  }
  t.idx_k_pool = ik;
  float* scores = (float*)dalloc(R * MAXB * 4);

  if (mode == "decode") {
    uint16_t* q = (uint16_t*)dalloc(R * Hq * 128 * 2);
    hipLaunchKernelGGL(fill_u16, dim3(256), dim3(256), 0, 0, q, R * Hq * 128, (uint16_t)0x3F80);
    t.q = q;
    void* kp = dalloc(rows * kv_row);
    void* vp = dalloc(rows * kv_row);
    if (kvc == MSA_DTYPE_BF16) {
      hipLaunchKernelGGL(fill_u16, dim3(4096), dim3(256), 0, 0, (uint16_t*)kp, rows * 128,
                         (uint16_t)0x3F80);
      hipLaunchKernelGGL(fill_u16, dim3(4096), dim3(256), 0, 0, (uint16_t*)vp, rows * 128,
                         (uint16_t)0x3F80);
    } else if (kvc == MSA_DTYPE_FP8_E4M3) {
      CHECK(hipMemset(kp, 0x38, rows * kv_row));
      CHECK(hipMemset(vp, 0x38, rows * kv_row));
      float* ks = (float*)dalloc(rows * 4);
      float* vs = (float*)dalloc(rows * 4);
      hipLaunchKernelGGL(fill_f32, dim3(1024), dim3(256), 0, 0, ks, rows, 1.0f);
      hipLaunchKernelGGL(fill_f32, dim3(1024), dim3(256), 0, 0, vs, rows, 1.0f);
      t.k_scale = ks;
      t.v_scale = vs;
    } else {
      CHECK(hipMemset(kp, 0x22, rows * kv_row));  // e2m1 1.0 in both nibbles
      CHECK(hipMemset(vp, 0x22, rows * kv_row));
      void* ks = dalloc(rows * 8);
      void* vs = dalloc(rows * 8);
      CHECK(hipMemset(ks, 0x38, rows * 8));  // e4m3 1.0
      CHECK(hipMemset(vs, 0x38, rows * 8));
      t.k_scale = ks;
      t.v_scale = vs;
    }
    t.k_pool = kp;
    t.v_pool = vp;
  }
  CHECK(hipDeviceSynchronize());

  void* ws = nullptr;
  float* out = nullptr;
  size_t ws_bytes = 0;
  if (mode == "decode") {
    ws_bytes = msa_workspace_bytes(&p);
    ws = dalloc(ws_bytes);
    out = (float*)dalloc(R * Hq * 128 * 4);
  }
  const size_t flush_bytes = (size_t)1 << 30;
  void* flush_a = flush ? dalloc(flush_bytes) : nullptr;
  void* flush_b = flush ? dalloc(flush_bytes) : nullptr;
  for (int i = 0; i < launches; ++i) {
    if (flush)
      hipLaunchKernelGGL(copy16, dim3(4096), dim3(256), 0, 0, (const u32x4*)flush_a,
                         (u32x4*)flush_b, flush_bytes / 16);
    const int st = mode == "scan" ? msa_index_score(&p, &t, scores, nullptr)
                                  : msa_decode(&p, &t, nullptr, nullptr, out, ws, ws_bytes, nullptr);
    if (st != MSA_OK) {
      fprintf(stderr, "%s failed: %s\n", mode.c_str(), msa_status_string(st));
      return 1;
    }
  }
  CHECK(hipDeviceSynchronize());
  char rec[512];
  msa_last_dispatch(rec, sizeof(rec));
  size_t idx_bytes = 0;
  // per (token, index head): 64 elements, plus 4 scale codes for 4-bit keys
  const size_t tok_bytes = idc == MSA_DTYPE_NVFP4 ? 32 + 4 : 64 * ie;
  for (int b = 0; b < B; ++b) idx_bytes += (size_t)((ctx[b] + 127) / 128) * Hidx * 128 * tok_bytes;
  printf("%s launches %d index_key_bytes_per_launch %zu dispatch %s\n", mode.c_str(), launches,
         idx_bytes, rec);
  return 0;
}
