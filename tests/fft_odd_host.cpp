// Host harness for the odd-length register DFTs of csrc/fft_odd.hpp: reads
// `count` complex vectors of length N (float32 pairs) from a file, applies
// the forward (inv = 0) or unnormalised inverse (inv = 1) DFT and writes the
// results.  Built and driven by tests/test_fft_odd.py.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fft_odd.hpp"

using namespace hyena;

template <int N, bool INV>
static int run(const char* in, const char* out, long count) {
  std::vector<cf> v((size_t)count * N);
  FILE* f = fopen(in, "rb");
  if (!f || fread(v.data(), sizeof(cf), v.size(), f) != v.size()) return 2;
  fclose(f);
  for (long c = 0; c < count; ++c) RegDft<N, INV>::run(v.data() + (size_t)c * N);
  f = fopen(out, "wb");
  if (!f || fwrite(v.data(), sizeof(cf), v.size(), f) != v.size()) return 3;
  fclose(f);
  return 0;
}

template <int N>
static int dispatch_dir(int inv, const char* in, const char* out, long count) {
  return inv ? run<N, true>(in, out, count) : run<N, false>(in, out, count);
}

int main(int argc, char** argv) {
  if (argc != 6) {
    fprintf(stderr, "usage: %s N inv in out count\n", argv[0]);
    return 1;
  }
  const int n = atoi(argv[1]), inv = atoi(argv[2]);
  const long count = atol(argv[5]);
  switch (n) {
    case 3: return dispatch_dir<3>(inv, argv[3], argv[4], count);
    case 5: return dispatch_dir<5>(inv, argv[3], argv[4], count);
    case 9: return dispatch_dir<9>(inv, argv[3], argv[4], count);
    case 15: return dispatch_dir<15>(inv, argv[3], argv[4], count);
    case 25: return dispatch_dir<25>(inv, argv[3], argv[4], count);
    case 27: return dispatch_dir<27>(inv, argv[3], argv[4], count);
  }
  fprintf(stderr, "unsupported length %d\n", n);
  return 1;
}
