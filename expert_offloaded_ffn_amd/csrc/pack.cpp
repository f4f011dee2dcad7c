// moe_pack_expert: writes one expert bundle in the layout the kernels read.
//
// The bundle is the unit of residency: an expert's three matrices and, for
// fp8, their block scales travel together ("Running 35B MoE Models on 8GB
// GPUs", section "Technical Insight": quantisation scales belong to the atomic
// cache unit). Pure host code.
#include <cmath>
#include <cstring>

#include "moe_internal.h"

namespace {

inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

// Byte offsets of the MXFP4 bundle's four regions (codes and scales of W_gu, then of W_dn).
struct BundleGeomView {
  size_t gu, gs, dn, ds;
};
inline BundleGeomView bundle_view(int d, int F) {
  BundleGeomView g;
  g.gu = 0;
  g.gs = al256((size_t)2 * F * d / 2);
  g.dn = g.gs + al256((size_t)2 * F * (d / 32));
  g.ds = g.dn + al256((size_t)d * F / 2);
  return g;
}

// Row R of the interleaved [2F, K] gate/up matrix -> (is_up, hidden column).
inline void gu_row(int R, bool* up, int* col) {
  const int j = R / 32, rr = R % 32;
  *up = rr >= 16;
  *col = 16 * j + (rr & 15);
}

// bf16/f32 element copy helpers
template <typename T>
inline T at(const void* p, size_t i) { return static_cast<const T*>(p)[i]; }

// Tiled store of an [N, K] matrix given by get(n, k). bf16: 1 KiB tiles of 16 x 32, lane
// l's 8 elements (row l%16, columns 8*(l/16)..+7) at 16*l. fp8: 2 KiB tiles of 16 x 128
// in two 1 KiB halves; byte h*1024 + 16*l + b holds row l%16, column 32*(l/16) + 16h + b.
template <typename T, int TK, typename Get>
void store_tiled(char* dst, int N, int K, Get get) {
  const int tiles_k = K / TK;
  const int per_lane = TK / 4;  // elements per lane: 8 (bf16, TK=32) or 32 (fp8, TK=128)
  for (int nb = 0; nb < N / 16; ++nb)
    for (int kb = 0; kb < tiles_k; ++kb) {
      T* tile = reinterpret_cast<T*>(dst + ((size_t)nb * tiles_k + kb) * 1024 * (TK == 32 ? 1 : 2));
      for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < per_lane; ++i) {
          const int n = nb * 16 + (lane & 15);
          const int k = kb * TK + per_lane * (lane >> 4) + i;
          const size_t pos = TK == 32 ? (size_t)lane * 8 + i : (size_t)(i >> 4) * 1024 + lane * 16 + (i & 15);
          tile[pos] = get(n, k);
        }
    }
}

// MXFP4 store of an [N, K] matrix: codes get(n, k) (0..15) two per byte in 16 x 128 chunks
// (byte 16*l + 4*c + j of a chunk: row l%16, columns 32c + 8*(l/16) + 2j, low nibble, and
// + 1, high nibble) and E8M0 exponents esc(n, kb) of 32-column blocks, 64 bytes per chunk
// (byte 4r + c: row r, block 4 kc + c).
template <typename GetCode, typename GetExp>
void store_mxfp4(char* codes, char* scales, int N, int K, GetCode get, GetExp esc) {
  const int KC = K / 128;
  for (int nb = 0; nb < N / 16; ++nb)
    for (int kc = 0; kc < KC; ++kc) {
      uint8_t* ch = reinterpret_cast<uint8_t*>(codes + ((size_t)nb * KC + kc) * 1024);
      uint8_t* sc = reinterpret_cast<uint8_t*>(scales + ((size_t)nb * KC + kc) * 64);
      for (int lane = 0; lane < 64; ++lane)
        for (int c = 0; c < 4; ++c)
          for (int j = 0; j < 4; ++j) {
            const int n = nb * 16 + (lane & 15);
            const int k = kc * 128 + 32 * c + 8 * (lane >> 4) + 2 * j;
            ch[16 * lane + 4 * c + j] = (uint8_t)((get(n, k) & 15) | ((get(n, k + 1) & 15) << 4));
          }
      for (int r = 0; r < 16; ++r)
        for (int c = 0; c < 4; ++c) sc[4 * r + c] = esc(nb * 16 + r, 4 * kc + c);
    }
}

// E8M0 exponent of a power of two 2^(e-127), e in 0..254, or -1.
int e8m0_of(float s) {
  if (!(s > 0.f)) return -1;
  int ex;
  const float m = std::frexp(s, &ex);   // s = m * 2^ex, m in [0.5, 1)
  if (m != 0.5f) return -1;
  const int e = ex - 1 + 127;
  return (e >= 0 && e <= 254) ? e : -1;
}

}  // namespace

using namespace moeffn;

extern "C" moe_status moe_pack_expert(int32_t d, int32_t F, int32_t w_dtype, const void* wg, const void* wu,
                                      const void* wd, const float* sg, const float* su, const float* sd,
                                      void* bundle_host) {
  clear_error();
  const size_t bytes = moe_bundle_bytes(d, F, w_dtype);
  MOE_REQUIRE(bytes > 0, MOE_EINVAL, "moe_pack_expert: unsupported sizes d=%d F=%d for w_dtype %d", d, F, w_dtype);
  MOE_REQUIRE(wg && wu && wd && bundle_host, MOE_EINVAL, "moe_pack_expert: NULL argument");
  char* out = static_cast<char*>(bundle_host);
  std::memset(out, 0, bytes);
  if (w_dtype == MOE_F32) {
    float* g = reinterpret_cast<float*>(out);
    float* u = g + (size_t)F * d;
    float* dn = reinterpret_cast<float*>(out + al256((size_t)2 * F * d * 4));
    for (int i = 0; i < d; ++i)
      for (int f = 0; f < F; ++f) {
        g[(size_t)f * d + i] = at<float>(wg, (size_t)i * F + f);
        u[(size_t)f * d + i] = at<float>(wu, (size_t)i * F + f);
      }
    for (int f = 0; f < F; ++f)
      for (int c = 0; c < d; ++c) dn[(size_t)c * F + f] = at<float>(wd, (size_t)f * d + c);
    return MOE_OK;
  }
  if (w_dtype == MOE_BF16) {
    store_tiled<uint16_t, 32>(out, 2 * F, d, [&](int n, int k) {
      bool up; int col; gu_row(n, &up, &col);
      return at<uint16_t>(up ? wu : wg, (size_t)k * F + col);
    });
    char* dn = out + al256((size_t)2 * F * d * 2);
    store_tiled<uint16_t, 32>(dn, d, F, [&](int n, int k) { return at<uint16_t>(wd, (size_t)k * d + n); });
    return MOE_OK;
  }
  if (w_dtype == MOE_MXFP4) {
    MOE_REQUIRE(sg && su && sd, MOE_EINVAL, "moe_pack_expert: mxfp4 needs the three scale grids");
    const uint8_t* cg = static_cast<const uint8_t*>(wg);
    const uint8_t* cu = static_cast<const uint8_t*>(wu);
    const uint8_t* cd = static_cast<const uint8_t*>(wd);
    for (size_t i = 0; i < (size_t)d * F; ++i)
      MOE_REQUIRE(cg[i] < 16 && cu[i] < 16 && cd[i] < 16, MOE_EINVAL, "moe_pack_expert: mxfp4 code above 15");
    for (size_t i = 0; i < (size_t)(d / 32) * F; ++i)
      MOE_REQUIRE(e8m0_of(sg[i]) >= 0 && e8m0_of(su[i]) >= 0, MOE_EINVAL,
                  "moe_pack_expert: mxfp4 scales must be powers of two 2^(e-127), e in 0..254");
    for (size_t i = 0; i < (size_t)(F / 32) * d; ++i)
      MOE_REQUIRE(e8m0_of(sd[i]) >= 0, MOE_EINVAL,
                  "moe_pack_expert: mxfp4 scales must be powers of two 2^(e-127), e in 0..254");
    const BundleGeomView g = bundle_view(d, F);
    // W_gu [2F, d]: row R -> gate or up column; the scale grids are [d/32][F]
    store_mxfp4(out + g.gu, out + g.gs, 2 * F, d,
                [&](int n, int k) { bool up; int col; gu_row(n, &up, &col); return (up ? cu : cg)[(size_t)k * F + col]; },
                [&](int n, int kb) {
                  bool up; int col; gu_row(n, &up, &col);
                  return (uint8_t)e8m0_of((up ? su : sg)[(size_t)kb * F + col]);
                });
    // W_dn [d, F]: row n = W_down column n; scales [F/32][d]
    store_mxfp4(out + g.dn, out + g.ds, d, F, [&](int n, int k) { return cd[(size_t)k * d + n]; },
                [&](int n, int kb) { return (uint8_t)e8m0_of(sd[(size_t)kb * d + n]); });
    return MOE_OK;
  }
  // fp8 e4m3 codes with 128x128 block scales
  MOE_REQUIRE(sg && su && sd, MOE_EINVAL, "moe_pack_expert: fp8 needs the three scale grids");
  store_tiled<uint8_t, 128>(out, 2 * F, d, [&](int n, int k) {
    bool up; int col; gu_row(n, &up, &col);
    return at<uint8_t>(up ? wu : wg, (size_t)k * F + col);
  });
  const size_t dn_off = al256((size_t)2 * F * d);
  store_tiled<uint8_t, 128>(out + dn_off, d, F, [&](int n, int k) { return at<uint8_t>(wd, (size_t)k * d + n); });
  const int db = d / 128, fb = F / 128;
  float* s_g = reinterpret_cast<float*>(out + dn_off + al256((size_t)d * F));
  float* s_u = reinterpret_cast<float*>(reinterpret_cast<char*>(s_g) + al256((size_t)fb * db * 4));
  float* s_d = reinterpret_cast<float*>(reinterpret_cast<char*>(s_u) + al256((size_t)fb * db * 4));
  for (int fi = 0; fi < fb; ++fi)
    for (int di = 0; di < db; ++di) {
      s_g[fi * db + di] = sg[di * fb + fi];   // input grids are [in/128][out/128]
      s_u[fi * db + di] = su[di * fb + fi];
      s_d[di * fb + fi] = sd[fi * db + di];
    }
  return MOE_OK;
}
