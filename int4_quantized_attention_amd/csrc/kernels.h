// Kernel argument blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

struct Shape {
  int B, H, F, Hs, Ws, D, Df, Dh, Dw, qk_blk, kv_blk;
};

constexpr int kTokenPad = 256;   // code tensors hold Np = N rounded up to this
constexpr int kMaxBatch = 64;    // batch elements of a variable-length call
constexpr int kMaxHeads = 512;   // heads per attention launch (more -> several launches)
constexpr int kMaxDevices = 64;  // devices the no-allocation entry point keeps a scratch address for
constexpr size_t kQuantScratchBytes = (size_t)64 << 20;  // its fixed scratch per device

struct QuantArgs {
  Shape s;
  int64_t Np;
  int rot, smooth;
  int smooth_q;   // Q minus its channel mean; the per-key term goes to kbias
  const void* q;
  const void* k;
  const void* v;
  const float* table;
  uint8_t* qc;
  float* qs;
  uint8_t* kc;
  float* ks;
  uint8_t* vc;
  float* vs;
  int32_t* vcol;
  float* kbias;  // [B,H,Np] mu_q . K_j (smooth_q only)
  int nlens;     // 0, or B: lens[b] tokens of batch element b exist (variable-length batch)
  int lens[kMaxBatch];
  // workspace
  double* kpart;
  double* qpart;
  float* kmu;
  float* qmu;
  uint32_t* vamax;
};

struct AttnArgs {
  const uint8_t* qc;
  const float* qs;
  const uint8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  uint8_t* img;   // workspace: per-group LDS images of K (packed fp6) and V^T (fp8)
  int64_t img_bytes;  // its size (images that would not fit are neither written nor read)
  void* out;
  int out_kind;  // 0 binary32, 1 binary16, 2 bfloat16
  int64_t N, Np;
  int qk_blk;
  int nqt, total, per_xcd;
  float C0, L15;  // L15: fl(log2 15), or fl(log2 7) for the symmetric-P baseline
  int p_zero;       // zero point of the dumped P codes: 8 (range-rectified) or 0
  int causal;       // 0 bidirectional; c > 0: query i sees key j iff j / c <= i / c (c < N)
  const float* kbias;  // nullable [B,H,Np]: per-key score term left by Q smoothing
  int H;               // heads per batch element (for lens)
  int nlens;           // 0, or B: lens[b] tokens of batch element b exist
  int lens[kMaxBatch];
  float T[16];  // P level thresholds (15 used)
  unsigned long long* stats;  // nullable device u64[5]: skip counters, added to
  // debug (rows [dbg_row0, dbg_row0 + dbg_n) of the single listed head)
  int dbg_row0, dbg_n;
  int32_t* dbg_aqk;
  int8_t* dbg_p;
  int32_t* dbg_apv;
  float* dbg_m;
  float* dbg_l;
  int nheads;
  int heads[kMaxHeads];
};

struct FbArgs {
  Shape s;
  int64_t N, Np;
  const void* q;
  const void* k;
  const void* v;
  const float* table;
  _Float16* qr;     // workspace: RoPE'd Q  [B*H][Np][D] f16
  uint8_t* img;     // workspace: per head, one LDS image per 64-key group (fallback_image_bytes(D) each)
  int64_t img_bytes;  // bytes of the image region
  void* out;
  int out_kind;  // 0 binary32, 1 binary16, 2 bfloat16
  int nqt, total, per_xcd;
  float scale_log2;  // log2(e) / sqrt(D)
  int causal;        // 0 bidirectional; c > 0: query i sees key j iff j / c <= i / c (c < N)
  int nlens;         // 0, or B: lens[b] tokens of batch element b exist
  int lens[kMaxBatch];
  int nheads;
  int heads[kMaxHeads];
};

struct LevelTable {
  float T[17];  // the 15 P level thresholds, then +inf, +inf
};

hipError_t launch_quantize(const QuantArgs& a, int dtype, hipStream_t st);
// the device address of this device's kQuantScratchBytes of library scratch
hipError_t quant_scratch(void** out);
// out[i] = the attention's P level decision for y = bits first + i (low nibble) and
// the exact fix alone (high nibble), i < n
hipError_t launch_level_probe(uint32_t first, int64_t n, uint8_t* out, const float* thresholds15,
                              hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, int D, int kv_blk, bool dbg, hipStream_t st);
// bytes of the attention workspace: the per-group LDS images of every head (the
// image geometry lives with the kernel; D, kv_blk, qk_blk as validated by the API)
size_t attention_workspace_bytes(int D, int kv_blk, int qk_blk, int64_t BH, int64_t Np);
hipError_t launch_fallback_prep(const FbArgs& a, int dtype, hipStream_t st);
hipError_t launch_fallback(const FbArgs& a, hipStream_t st);
// bytes of one 64-key group's LDS image of the fallback (K rows, then V^T rows)
size_t fallback_image_bytes(int D);

}  // namespace ra
