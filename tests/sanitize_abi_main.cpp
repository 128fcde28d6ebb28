// Host sanitizer driver for the C ABI (tests/test_sanitizers_cpu.py builds
// libdsa's sources with the host side under -fsanitize=address,undefined and
// runs this). It fuzzes every entry point's host path -- validation, the
// workspace-size arithmetic and the launch planning -- with sizes drawn from
// edge values (0, 1, powers of two and their neighbours, INT_MAX) and NULL or
// dummy pointers. Dummy pointers are never dereferenced on the host. When no
// GPU is visible, calls that pass validation go on to plan their launches and
// fail at the first HIP call with DSA_ERR_HIP; when a GPU is visible only
// calls that fail validation (a NULL pointer) and the size queries run, so
// nothing is ever launched on dummy pointers.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dsa.h"

namespace {
uint64_t st = 0x9E3779B97F4A7C15ull;
uint64_t rnd() {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return st;
}
const int kVals[] = {-1, 0, 1, 2, 3, 15, 16, 17, 31, 32, 33, 48, 64, 96, 100, 127, 128, 129,
                     192, 255, 256, 257, 511, 512, 1000, 2047, 2048, 2049, 4096, 16384, 16385,
                     32768, 65535, 65536, 131072, 528385, 1 << 24, INT_MAX - 1, INT_MAX};
int iv() {
  if (rnd() % 4 == 0) return (int)(rnd() % 300);  // small sizes pass validation more often
  return kVals[rnd() % (sizeof kVals / sizeof kVals[0])];
}
float fv() {
  const float v[] = {0.125f, 1.0f, 0.0f, -1.0f, NAN, INFINITY, 1e-30f};
  return v[rnd() % 7];
}
void* dummy = reinterpret_cast<void*>(4096);
bool gpu_visible = false;
// a required pointer: NULL sometimes, and always NULL in one slot when a GPU is visible
const void* pv(int slot, int null_slot) {
  if (gpu_visible && slot == null_slot) return nullptr;
  return rnd() % 16 == 0 ? nullptr : dummy;
}
int bad = 0;
void expect(int status, const char* fn) {
  if (status < DSA_OK || status > DSA_ERR_HIP) {
    fprintf(stderr, "%s returned unknown status %d\n", fn, status);
    bad = 1;
  }
  if (gpu_visible && status == DSA_OK) {
    fprintf(stderr, "%s passed validation with a NULL pointer\n", fn);
    bad = 1;
  }
  if (status != DSA_OK && strlen(dsa_last_error()) == 0 && status != DSA_ERR_HIP) {
    fprintf(stderr, "%s: status %d without a message\n", fn, status);
    bad = 1;
  }
}
}  // namespace

#define P(i) pv(i, ns)
#define VP(i) const_cast<void*>(pv(i, ns))

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
  gpu_visible = ndev > 0;
  const int N = 4000;
  for (int it = 0; it < N; ++it) {
    const int ns = (int)(rnd() % 3);  // which pointer is NULL when a GPU is visible
    int ws = 0;
    size_t wsb = (size_t)iv() * (size_t)(rnd() % 4096);
    (void)dsa_topk_workspace_size(iv(), iv(), iv(), iv());
    (void)dsa_sparse_attn_prefill_workspace_size(iv(), iv(), iv(), iv(), iv(), iv(), iv(), iv() & 1);
    (void)dsa_sparse_attn_prefill_pas_workspace_size(iv(), iv(), iv(), iv(), iv(), iv(), iv(), iv(),
                                                     iv() & 1);
    (void)dsa_sparse_attn_decode_workspace_size(iv(), iv(), iv(), iv());
    (void)dsa_sparse_attn_decode_pas_workspace_size(iv(), iv(), iv(), iv(), iv());
    (void)swa_attn_workspace_size(iv(), iv(), iv(), iv(), iv(), iv(), iv() & 1);
    (void)swa_attn_pas_workspace_size(iv(), iv(), iv(), iv(), iv(), iv(), iv(), iv() & 1);
    (void)swa_attn_gqa_workspace_size(iv(), iv(), iv(), iv(), iv(), iv(), iv() & 1);
    (void)dsa_indexer_prologue_workspace_size(iv(), iv(), iv());
    {
      int a, b, c, tab[260];
      expect(dsa_prefill_work_plan(iv(), iv(), iv(), iv(), iv(), iv(), iv(), &a, &b, &c, tab,
                                   (int)(rnd() % 260)),
             "dsa_prefill_work_plan");
    }
    (void)ws;
    const int dt = (int)(rnd() % 3);
    expect(dsa_index_scores(P(0), P(1), P(2), (float*)VP(0), iv(), iv(), iv(), iv(), iv(), iv(),
                            fv(), (int)(rnd() % 4), dt, nullptr),
           "dsa_index_scores");
    expect(dsa_index_quant_fp8(P(0), (uint8_t*)VP(1), (float*)VP(2), (long long)iv() * iv(), iv(),
                               dt, nullptr),
           "dsa_index_quant_fp8");
    expect(dsa_index_scores_fp8((const uint8_t*)P(0), (const float*)P(1), (const uint8_t*)P(2),
                                (const float*)P(0), P(1), (float*)VP(2), iv(), iv(), iv(), iv(),
                                iv(), iv(), fv(), (int)(rnd() % 4), dt, nullptr),
           "dsa_index_scores_fp8");
    // (the top-k calls have two required pointers; the workspace may be NULL)
    const float* tsc = (const float*)pv(0, ns % 2);
    int32_t* tix = (int32_t*)const_cast<void*>(pv(1, ns % 2));
    void* tws = rnd() % 2 ? dummy : nullptr;
    expect(dsa_topk(tsc, tix, iv(), iv(), iv(), iv(), tws, wsb, nullptr), "dsa_topk");
    expect(dsa_topk_unsorted(tsc, tix, iv(), iv(), iv(), iv(), tws, wsb, nullptr),
           "dsa_topk_unsorted");
    (void)dsa_index_topk_workspace_size(iv(), iv(), iv(), iv());
    expect(dsa_index_topk(P(0), P(1), P(2), tix, iv(), iv(), iv(), iv(), iv(), iv(), fv(),
                          (int)(rnd() % 4), dt, iv(), (int)(rnd() % 3), tws, wsb, nullptr),
           "dsa_index_topk");
    const int B = iv(), S = iv(), T = iv(), past = iv(), H = iv();
    expect(dsa_sparse_attn_prefill(P(0), P(1), P(2), (const int32_t*)P(0), P(1), VP(2), B, S, T,
                                   past, H, iv(), iv(), iv(), iv(), fv(), (int)(rnd() % 3), dt,
                                   VP(0), wsb, nullptr),
           "dsa_sparse_attn_prefill");
    expect(dsa_sparse_attn_prefill_pas(P(0), P(1), P(2), P(0), P(1), iv(), (const int32_t*)P(2),
                                       P(0), VP(1), B, S, T, past, H, iv(), iv(), iv(), iv(),
                                       fv(), (int)(rnd() % 3), dt, VP(2), wsb, nullptr),
           "dsa_sparse_attn_prefill_pas");
    expect(dsa_sparse_attn_decode(P(0), P(1), P(2), (const int32_t*)P(0), P(1), VP(2), B, T, H,
                                  iv(), iv(), iv(), iv(), fv(), (int)(rnd() % 3), dt, VP(0), wsb,
                                  nullptr),
           "dsa_sparse_attn_decode");
    expect(dsa_sparse_attn_decode_pas(P(0), P(1), P(2), P(0), P(1), iv(), (const int32_t*)P(2),
                                      P(0), VP(1), B, T, H, iv(), iv(), iv(), iv(), fv(),
                                      (int)(rnd() % 3), dt, VP(2), wsb, nullptr),
           "dsa_sparse_attn_decode_pas");
    expect(swa_attn(P(0), P(1), P(2), P(0), VP(1), B, S, T, past, iv(), H, iv(), iv(), iv(), iv(),
                    fv(), (int)(rnd() % 3), dt, VP(2), wsb, nullptr),
           "swa_attn");
    expect(swa_attn_pas(P(0), P(1), P(2), P(0), P(1), iv(), P(2), VP(0), B, S, T, past, iv(), H,
                        iv(), iv(), iv(), iv(), fv(), (int)(rnd() % 3), dt, VP(1), wsb, nullptr),
           "swa_attn_pas");
    expect(swa_attn_gqa(P(0), P(1), P(2), P(0), VP(1), B, S, T, past, iv(), H, iv(), iv(), iv(),
                        iv(), iv(), fv(), (int)(rnd() % 3), dt, VP(2), wsb, nullptr),
           "swa_attn_gqa");
    expect(dsa_indexer_prologue(P(0), P(1), P(2), P(0), P(1), P(2), P(0), (const float*)P(1),
                                (const float*)P(2), VP(0), VP(1), VP(2), B, S, T, past, iv(), iv(),
                                iv(), iv(), iv(), fv(), dt, VP(0), wsb, nullptr),
           "dsa_indexer_prologue");
    (void)dsa_mla_prologue_workspace_size(iv(), iv(), iv());
    expect(dsa_mla_prologue(P(0), P(1), P(2), P(0), P(1), P(2), (const float*)P(0),
                            (const float*)P(1), VP(2), VP(0), VP(1), VP(2), B, S, T, past, iv(),
                            iv(), iv(), iv(), H, iv(), iv(), iv(), dt, VP(0), wsb, nullptr),
           "dsa_mla_prologue");
  }
  for (int s = -2; s < 8; ++s) (void)dsa_status_string(s);
  if (bad) return 3;
  printf("abi sanitizer driver: ok (%d rounds, GPU %s)\n", N, gpu_visible ? "visible" : "absent");
  return 0;
}
