// Driver for the sanitizer build of the library's host routines (packers,
// uniform rewrite, quantizer, footprint and group search). Built with g++ and
// -fsanitize=address,undefined by tests/test_sanitize_host.py, linked against
// the host sources only (no HIP). For every case listed in <dir>/cases.txt it
// reads the inputs the test wrote, runs the routine on buffers sized exactly
// as the size queries say (so any overrun is caught), writes the outputs back,
// and checks the error paths (null pointers, short buffers) return their codes.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "lutgemm.h"

namespace {

std::string g_dir;

template <class T>
std::vector<T> read_file(const std::string& name, size_t count) {
  std::vector<T> v(count);
  FILE* f = fopen((g_dir + "/" + name).c_str(), "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", name.c_str());
    exit(10);
  }
  if (count && fread(v.data(), sizeof(T), count, f) != count) {
    fprintf(stderr, "short read %s\n", name.c_str());
    exit(11);
  }
  fclose(f);
  return v;
}

template <class T>
void write_file(const std::string& name, const std::vector<T>& v) {
  FILE* f = fopen((g_dir + "/" + name).c_str(), "wb");
  if (!f || (v.size() && fwrite(v.data(), sizeof(T), v.size(), f) != v.size())) exit(12);
  fclose(f);
}

int g_fail = 0;

void expect(int got, int want, const char* what, int idx) {
  if (got != want) {
    fprintf(stderr, "case %d: %s returned %d, expected %d\n", idx, what, got, want);
    g_fail = 1;
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  g_dir = argv[1];
  FILE* cf = fopen((g_dir + "/cases.txt").c_str(), "r");
  if (!cf) return 3;
  char kind[32];
  int idx, N, K, q, g, off, iters;
  while (fscanf(cf, "%d %31s %d %d %d %d %d %d", &idx, kind, &N, &K, &q, &g, &off, &iters) == 8) {
    lutgemm_shape s;
    s.N = N;
    s.K = K;
    s.q = q;
    s.g = g;
    s.has_offset = off;
    const std::string pre = "c" + std::to_string(idx) + "_";
    size_t nb = 0, na = 0, no = 0;
    expect(lutgemm_packed_sizes(&s, &nb, &na, &no), LUTGEMM_OK, "lutgemm_packed_sizes", idx);
    const size_t G = K ? (size_t)K / g : 0;
    std::vector<uint8_t> ob(nb);
    std::vector<uint16_t> oa(na), oo(no);
    if (strcmp(kind, "pack") == 0) {
      auto bits = read_file<uint8_t>(pre + "bits.bin", (size_t)q * N * (K / 8));
      auto alpha = read_file<uint16_t>(pre + "alpha.bin", (size_t)q * N * G);
      std::vector<uint16_t> offset = off ? read_file<uint16_t>(pre + "offset.bin", (size_t)N * G)
                                         : std::vector<uint16_t>();
      const uint16_t* op = off ? offset.data() : nullptr;
      expect(bcq_pack(&s, bits.data(), alpha.data(), op, ob.data(), nb, oa.data(), na,
                      off ? oo.data() : nullptr, no),
             LUTGEMM_OK, "bcq_pack", idx);
      if (nb) {
        expect(bcq_pack(&s, bits.data(), alpha.data(), op, ob.data(), nb - 1, oa.data(), na,
                        off ? oo.data() : nullptr, no),
               LUTGEMM_ERR_BUFFER, "bcq_pack (short bits)", idx);
        expect(bcq_pack(&s, nullptr, alpha.data(), op, ob.data(), nb, oa.data(), na,
                        off ? oo.data() : nullptr, no),
               LUTGEMM_ERR_NULL, "bcq_pack (null bits)", idx);
      }
    } else if (strcmp(kind, "uniform") == 0) {
      auto codes = read_file<uint8_t>(pre + "codes.bin", (size_t)N * K);
      auto scale = read_file<uint16_t>(pre + "scale.bin", (size_t)N * G);
      auto zero = read_file<uint8_t>(pre + "zero.bin", (size_t)N * G);
      size_t n_rounded = 0;
      expect(bcq_pack_uniform(&s, codes.data(), scale.data(), zero.data(), ob.data(), nb,
                              oa.data(), na, oo.data(), no, &n_rounded),
             LUTGEMM_OK, "bcq_pack_uniform", idx);
      write_file(pre + "nrounded.bin", std::vector<uint64_t>{(uint64_t)n_rounded});
      if (na)
        expect(bcq_pack_uniform(&s, codes.data(), scale.data(), zero.data(), ob.data(), nb,
                                oa.data(), na - 1, oo.data(), no, &n_rounded),
               LUTGEMM_ERR_BUFFER, "bcq_pack_uniform (short alpha)", idx);
    } else if (strcmp(kind, "quantize") == 0) {
      auto w = read_file<uint16_t>(pre + "w.bin", (size_t)N * K);
      std::vector<uint8_t> bits((size_t)q * N * (K / 8));
      std::vector<uint16_t> alpha((size_t)q * N * G);
      double err = 0;
      expect(bcq_quantize(&s, w.data(), iters, bits.data(), bits.size(), alpha.data(),
                          alpha.size(), &err),
             LUTGEMM_OK, "bcq_quantize", idx);
      write_file(pre + "qbits.bin", bits);
      write_file(pre + "qalpha.bin", alpha);
      write_file(pre + "qerr.bin", std::vector<double>{err});
      if (!bits.empty())
        expect(bcq_quantize(&s, w.data(), iters, bits.data(), bits.size() - 1, alpha.data(),
                            alpha.size(), &err),
               LUTGEMM_ERR_BUFFER, "bcq_quantize (short bits)", idx);
    } else if (strcmp(kind, "footprint") == 0) {
      uint64_t fb = 0;
      expect(bcq_footprint_bits(&s, &fb), LUTGEMM_OK, "bcq_footprint_bits", idx);
      int32_t gs[8];
      uint64_t bs[8];
      expect(bcq_search_group_sizes(N, K, off, (double)iters / 8.0, gs, bs), LUTGEMM_OK,
             "bcq_search_group_sizes", idx);
      std::vector<uint64_t> out{fb};
      for (int i = 0; i < 8; ++i) out.push_back((uint64_t)gs[i]);
      for (int i = 0; i < 8; ++i) out.push_back(bs[i]);
      write_file(pre + "foot.bin", out);
    } else {
      return 4;
    }
    write_file(pre + "pbits.bin", ob);
    write_file(pre + "palpha.bin", oa);
    write_file(pre + "poffset.bin", oo);
  }
  fclose(cf);
  printf("%s\n", g_fail ? "FAIL" : "OK");
  return g_fail;
}
