// Test driver: runs every entry point of the CPU oracle on small, ragged inputs so
// that an AddressSanitizer / UndefinedBehaviorSanitizer build of the oracle can
// check its raw-pointer indexing.  Built and run by tests/test_oracle_sanitized.py
// (host code only; links oracle/rotattn_oracle.cpp directly).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
int64_t orc_table_entries(const int32_t* shp);
void orc_rope_table(const int32_t* shp, int32_t rot, double base, float* out);
void orc_rope_table_f64(const int32_t* shp, int32_t rot, double base, double* out);
void orc_rope_rotate(const int32_t* shp, int32_t rot, const float* tab, const float* x, float* out);
void orc_rope_rotate_f64(const int32_t* shp, int32_t rot, const double* tab, const double* x, double* out);
void orc_quantize_x(const int32_t* shp, int32_t rot, const float* tab, int32_t flags, const float* q,
                    const float* k, const float* v, int8_t* qc, float* qs, int8_t* kc, float* ks, int8_t* vc,
                    float* vs, int32_t* vcol, float* q_rot, float* k_rot, float* k_mu, float* q_mu,
                    float* k_bias, const int32_t* seq_lens);
void orc_attention_x(const int32_t* shp, const int8_t* qc, const float* qs, const int8_t* kc, const float* ks,
                     const int8_t* vc, const float* vs, const int64_t* rows, int64_t n_rows, double* out,
                     int32_t* a_qk, int8_t* pcode, int32_t* a_pv, float* m_out, double* l_out, int32_t pmax,
                     int32_t causal_block, const float* k_bias, const int32_t* seq_lens);
void orc_exact_attention_x(const int32_t* shp, const double* tab64_plain, const float* q, const float* k,
                           const float* v, const int64_t* rows, int64_t n_rows, double* out,
                           int32_t causal_block, const int32_t* seq_lens);
void orc_fallback_attention_x(const int32_t* shp, const float* tab_plain, const float* q, const float* k,
                              const float* v, const int64_t* rows, int64_t n_rows, double* out,
                              int32_t causal_block, const int32_t* seq_lens);
void orc_p_thresholds(float* out15);
void orc_p_levels(const float* y, int64_t n, int8_t* r);
int64_t orc_p_level_bruteforce(float lo, float hi, float* first);
void orc_f32_to_f16(const float* x, int64_t n, uint16_t* out);
}

namespace {

// SplitMix64 (Steele, Lea and Flood 2014) -> uniform -> rough normal (sum of 4)
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  float normal() {
    double t = 0;
    for (int i = 0; i < 4; ++i) t += (double)(next() >> 11) * (1.0 / 9007199254740992.0) - 0.5;
    return (float)(t * 1.7320508);
  }
};

int run_case(int B, int H, int F, int Hs, int Ws, int D, int Df, int Dh, int Dw, int qk, int kv, int rot,
             int flags, bool varlen, int causal, int pmax) {
  const int32_t shp[11] = {B, H, F, Hs, Ws, D, Df, Dh, Dw, qk, kv};
  const int64_t N = (int64_t)F * Hs * Ws, BH = (int64_t)B * H, nqb = (N + qk - 1) / qk, nkb = (N + kv - 1) / kv;
  Rng rng{(uint64_t)(N * 131 + D * 7 + qk * 3 + kv + rot)};
  std::vector<float> q(BH * N * D), k(BH * N * D), v(BH * N * D);
  for (auto* t : {&q, &k, &v})
    for (auto& x : *t) x = 2.0f * rng.normal();
  const int64_t ne = orc_table_entries(shp);
  std::vector<float> tab(ne), tab0(ne);
  std::vector<double> tab64(ne);
  orc_rope_table(shp, rot, 10000.0, tab.data());
  orc_rope_table(shp, 0, 10000.0, tab0.data());
  orc_rope_table_f64(shp, 0, 10000.0, tab64.data());
  std::vector<float> rot_out(BH * N * D);
  orc_rope_rotate(shp, rot, tab.data(), q.data(), rot_out.data());
  std::vector<double> q64(q.begin(), q.end()), r64(BH * N * D);
  orc_rope_rotate_f64(shp, rot == 1 ? 0 : rot, tab64.data(), q64.data(), r64.data());
  std::vector<int32_t> lens(B);
  for (int b = 0; b < B; ++b) lens[b] = (int32_t)(varlen ? 1 + (rng.next() % N) : N);
  const int32_t* sl = varlen ? lens.data() : nullptr;
  std::vector<int8_t> qc(BH * N * D), kc(BH * N * D), vc(BH * N * D);
  std::vector<float> qs(BH * nqb), ks(BH * nqb), vs(BH * D), qr(BH * N * D), kr(BH * N * D), kmu(BH * D),
      qmu(BH * D), kb(BH * N);
  std::vector<int32_t> vcol(BH * nkb * D);
  orc_quantize_x(shp, rot, tab.data(), flags, q.data(), k.data(), v.data(), qc.data(), qs.data(), kc.data(),
                 ks.data(), vc.data(), vs.data(), vcol.data(), qr.data(), kr.data(), kmu.data(), qmu.data(),
                 (flags & 2) ? kb.data() : nullptr, sl);
  std::vector<int64_t> rows;
  for (int64_t bh = 0; bh < BH; ++bh) {
    const int64_t n = varlen ? lens[bh / H] : N;
    for (int64_t i = 0; i < n; i += 1 + n / 7) rows.push_back(bh * N + i);
    rows.push_back(bh * N + n - 1);
  }
  const int64_t R = (int64_t)rows.size();
  std::vector<double> out(R * D), l(R);
  std::vector<int32_t> aqk(R * N), apv(R * nkb * D);
  std::vector<int8_t> pc(R * N);
  std::vector<float> m(R);
  orc_attention_x(shp, qc.data(), qs.data(), kc.data(), ks.data(), vc.data(), vs.data(), rows.data(), R,
                  out.data(), aqk.data(), pc.data(), apv.data(), m.data(), l.data(), pmax, causal,
                  (flags & 2) ? kb.data() : nullptr, sl);
  orc_exact_attention_x(shp, tab64.data(), q.data(), k.data(), v.data(), rows.data(), R, out.data(), causal, sl);
  orc_fallback_attention_x(shp, tab0.data(), q.data(), k.data(), v.data(), rows.data(), R, out.data(), causal,
                           sl);
  for (double x : out)
    if (!std::isfinite(x)) return 1;
  return 0;
}

}  // namespace

int main() {
  int bad = 0;
  // B, H, F, Hs, Ws, D, Df, Dh, Dw, qk, kv, rot, flags, varlen, causal, pmax
  bad += run_case(1, 2, 2, 4, 4, 64, 24, 20, 20, 16, 16, 1, 1, false, 0, 15);
  bad += run_case(2, 1, 3, 5, 7, 64, 24, 20, 20, 32, 64, 2, 3, true, 0, 15);
  bad += run_case(1, 2, 2, 5, 9, 128, 44, 42, 42, 64, 128, 3, 1, false, 7, 7);
  bad += run_case(2, 2, 1, 3, 11, 128, 16, 56, 56, 1, 256, 2, 3, true, 5, 15);
  bad += run_case(1, 1, 1, 1, 1, 64, 24, 20, 20, 16, 16, 0, 0, false, 0, 15);
  float th[15];
  orc_p_thresholds(th);
  std::vector<float> y(4096);
  for (size_t i = 0; i < y.size(); ++i) y[i] = -8.0f + 12.0f * (float)i / (float)y.size();
  std::vector<int8_t> r(y.size());
  orc_p_levels(y.data(), (int64_t)y.size(), r.data());
  float first = 0.f;
  bad += orc_p_level_bruteforce(0.5f, 0.5001f, &first) != 0;
  std::vector<uint16_t> h(y.size());
  orc_f32_to_f16(y.data(), (int64_t)y.size(), h.data());
  std::printf(bad ? "sanitized oracle run: %d bad cases\n" : "sanitized oracle run: ok\n", bad);
  return bad ? 1 : 0;
}
