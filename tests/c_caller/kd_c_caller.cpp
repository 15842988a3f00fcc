// A plain C++ caller of the C ABI in include/kd_loss.h, without PyTorch: it
// allocates device memory with the HIP runtime, runs one forward and one
// backward of a tied-teacher bf16 problem on its own stream, and writes the
// results back to files. The GPU tests feed it the same inputs as the Python
// binding and require identical results.
//
//   kd_c_caller --version        print kd_version() (no GPU needed)
//   kd_c_caller DIR              DIR/meta.txt: "n d v temperature ignore_index chunk"
//                                DIR/hidden.bin, weight.bin, teacher_hidden.bin: raw bf16
//                                DIR/labels.bin: int64
//                                writes DIR/loss.bin, kl.bin, student_ce.bin, dh.bin, dw.bin
//                                (fp32) and prints "status <fwd> <bwd> flags <f>"
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kd_loss.h"

namespace {

bool read_file(const std::string& path, std::vector<uint8_t>& buf, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  buf.resize(bytes);
  const size_t got = std::fread(buf.data(), 1, bytes, f);
  std::fclose(f);
  return got == bytes;
}

bool write_file(const std::string& path, const void* data, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const size_t put = std::fwrite(data, 1, bytes, f);
  std::fclose(f);
  return put == bytes;
}

// Device buffers freed on every exit path.
struct Dev {
  std::vector<void*> ptrs;
  void* alloc(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes < 16 ? 16 : bytes) != hipSuccess) return nullptr;
    ptrs.push_back(p);
    return p;
  }
  ~Dev() {
    for (void* p : ptrs) (void)hipFree(p);
  }
};

#define CHECK_HIP(x)                                                  \
  do {                                                                \
    if ((x) != hipSuccess) {                                          \
      std::fprintf(stderr, "HIP call failed: %s (line %d)\n", #x, __LINE__); \
      return 3;                                                       \
    }                                                                 \
  } while (0)

int run(const std::string& dir) {
  long long n = 0, d = 0, v = 0, ignore = 0, chunk = 0;
  float temperature = 0.f;
  {
    FILE* f = std::fopen((dir + "/meta.txt").c_str(), "r");
    if (!f) return 2;
    const int got = std::fscanf(f, "%lld %lld %lld %f %lld %lld", &n, &d, &v, &temperature, &ignore, &chunk);
    std::fclose(f);
    if (got != 6 || n < 1 || d < 1 || v < 1) return 2;
  }
  const size_t hb = (size_t)n * d * 2, wb = (size_t)v * d * 2, lb = (size_t)n * 8;
  std::vector<uint8_t> h_s, h_t, w, lab;
  if (!read_file(dir + "/hidden.bin", h_s, hb) || !read_file(dir + "/teacher_hidden.bin", h_t, hb) ||
      !read_file(dir + "/weight.bin", w, wb) || !read_file(dir + "/labels.bin", lab, lb))
    return 2;

  CHECK_HIP(hipSetDevice(0));
  hipStream_t stream = nullptr;
  CHECK_HIP(hipStreamCreate(&stream));
  Dev dev;
  void* d_hs = dev.alloc(hb);
  void* d_ht = dev.alloc(hb);
  void* d_w = dev.alloc(wb);
  void* d_lab = dev.alloc(lb);
  float* d_loss = static_cast<float*>(dev.alloc(4));
  float* d_kl = static_cast<float*>(dev.alloc((size_t)n * 4));
  float* d_ce = static_cast<float*>(dev.alloc((size_t)n * 4));
  void* d_dh = dev.alloc((size_t)n * d * 4);
  void* d_dw = dev.alloc((size_t)v * d * 4);
  if (!d_hs || !d_ht || !d_w || !d_lab || !d_loss || !d_kl || !d_ce || !d_dh || !d_dw) return 3;
  CHECK_HIP(hipMemcpy(d_hs, h_s.data(), hb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_ht, h_t.data(), hb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w.data(), wb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_lab, lab.data(), lb, hipMemcpyHostToDevice));

  kd_student s;
  std::memset(&s, 0, sizeof(s));
  s.kind = KD_STUDENT_PROJECTION;
  s.dtype = KD_BF16;
  s.n = n;
  s.d = d;
  s.v = v;
  s.hidden = d_hs;
  s.weight = d_w;
  kd_teacher t;
  std::memset(&t, 0, sizeof(t));
  t.kind = KD_TEACHER_TIED;
  t.hidden = d_ht;
  kd_params p;
  std::memset(&p, 0, sizeof(p));
  p.student_ce_weight = 1.f;
  p.kl_weight = 1.f;
  p.temperature = temperature;
  p.ignore_index = ignore;
  p.reduction = KD_REDUCE_MEAN;
  p.vocab_chunk = chunk;
  p.kl_divergence = KD_KL_FORWARD;

  size_t ws_f = 0, ws_b = 0, saved_bytes = 0;
  kd_status st = kd_workspace_bytes(&s, &t, &p, 0, &ws_f);
  if (st == KD_OK) st = kd_workspace_bytes(&s, &t, &p, 1, &ws_b);
  if (st == KD_OK) st = kd_saved_bytes_for(&s, &t, &p, &saved_bytes);
  if (st != KD_OK) {
    std::printf("sizes failed: %s\n", kd_status_string(st));
    return 4;
  }
  void* ws_fwd = dev.alloc(ws_f);
  void* ws_bwd = dev.alloc(ws_b);
  void* saved = dev.alloc(saved_bytes);
  if (!ws_fwd || !ws_bwd || !saved) return 3;
  p.saved_bytes = (int64_t)saved_bytes;

  const kd_outputs out{d_loss, d_ce, nullptr, d_kl};
  const kd_status sf = kd_loss_fwd(&s, &t, &p, static_cast<const int64_t*>(d_lab), &out, saved, ws_fwd,
                                   ws_f, stream, nullptr);
  kd_status sb = KD_ERR_HIP;
  if (sf == KD_OK)
    sb = kd_loss_bwd(&s, &t, &p, static_cast<const int64_t*>(d_lab), saved, nullptr, d_dh, d_dw, 0,
                     ws_bwd, ws_b, stream, nullptr);
  int32_t flags = -1;
  if (sf == KD_OK) (void)kd_read_status(ws_fwd, stream, &flags);
  CHECK_HIP(hipStreamSynchronize(stream));

  std::vector<float> loss(1), kl((size_t)n), ce((size_t)n), dh((size_t)n * d), dw((size_t)v * d);
  CHECK_HIP(hipMemcpy(loss.data(), d_loss, 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(kl.data(), d_kl, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(ce.data(), d_ce, (size_t)n * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dh.data(), d_dh, dh.size() * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dw.data(), d_dw, dw.size() * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipStreamDestroy(stream));
  if (!write_file(dir + "/loss.bin", loss.data(), 4) || !write_file(dir + "/kl.bin", kl.data(), kl.size() * 4) ||
      !write_file(dir + "/student_ce.bin", ce.data(), ce.size() * 4) ||
      !write_file(dir + "/dh.bin", dh.data(), dh.size() * 4) ||
      !write_file(dir + "/dw.bin", dw.data(), dw.size() * 4))
    return 2;
  std::printf("status %d %d flags %d\n", (int)sf, (int)sb, (int)flags);
  return (sf == KD_OK && sb == KD_OK) ? 0 : 5;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc == 2 && std::strcmp(argv[1], "--version") == 0) {
    std::printf("%s\n", kd_version());
    return 0;
  }
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s --version | DIR\n", argv[0]);
    return 1;
  }
  return run(argv[1]);
}
