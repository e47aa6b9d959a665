// Drives the host layer of libfibatt (csrc/host.cpp) from a line protocol on
// stdin, for the CPU test that builds it under AddressSanitizer and
// UndefinedBehaviorSanitizer.  One request per line, one reply per line:
//   wythoff I             -> rc a b
//   modified I            -> rc a b
//   windows H WMIN WMAX   -> rc w_1 .. w_H
//   offsets H N CAP a.. b.. w..       -> rc head_ptr[0..H] ; offs..
//   desc B H N D DT a.. b.. w..       -> rc (fibatt_bwd_workspace_floats)
//   table B H N D DT CLS hp[0..H] offs..  -> rc (fibatt_bwd_table_workspace_floats)
//   layouts BWD B H N D DT sb sh sn x8    -> rc strided
// rc is the status code (or the workspace size, -1 on error).
#include <cstdint>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/fibatt.h"
#include "../../structured_sparse_head_amd/csrc/validate.h"

namespace {

std::vector<int32_t> read_ints(std::istringstream& in, int n) {
  std::vector<int32_t> v(n);
  for (int i = 0; i < n; ++i) in >> v[i];
  return v;
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    in >> op;
    if (op == "wythoff" || op == "modified") {
      int32_t i, a = -7, b = -7;
      in >> i;
      const int rc = op == "wythoff" ? fibatt_wythoff(i, &a, &b) : fibatt_wythoff_modified(i, &a, &b);
      std::cout << rc << " " << a << " " << b << "\n";
    } else if (op == "windows") {
      int32_t H, lo, hi;
      in >> H >> lo >> hi;
      std::vector<int32_t> w(H > 0 ? H : 1, -1);
      const int rc = fibatt_windows(H, lo, hi, H > 0 ? w.data() : nullptr);
      std::cout << rc;
      if (rc == FIBATT_OK)
        for (int32_t x : w) std::cout << " " << x;
      std::cout << "\n";
    } else if (op == "offsets") {
      int32_t H, N, cap;
      in >> H >> N >> cap;
      const auto a = read_ints(in, H), b = read_ints(in, H), w = read_ints(in, H);
      std::vector<int32_t> ptr(H + 1, -1), offs(cap > 0 ? cap : 1, -1);
      const int rc = fibatt_offsets(H, N, a.data(), b.data(), w.data(), ptr.data(),
                                    cap > 0 ? offs.data() : nullptr, cap);
      std::cout << rc;
      for (int32_t x : ptr) std::cout << " " << x;
      std::cout << " ;";
      if (rc == FIBATT_OK)
        for (int32_t i = 0; i < ptr[H]; ++i) std::cout << " " << offs[i];
      std::cout << "\n";
    } else if (op == "desc") {
      int32_t B, H, N, D, dt;
      in >> B >> H >> N >> D >> dt;
      const int n = H > 0 ? H : 0;
      const auto a = read_ints(in, n), b = read_ints(in, n), w = read_ints(in, n);
      const fibatt_desc d{B, H, N, D, dt, a.data(), b.data(), w.data()};
      std::cout << fibatt_bwd_workspace_floats(&d) << "\n";
    } else if (op == "table") {
      int32_t B, H, N, D, dt, cls;
      in >> B >> H >> N >> D >> dt >> cls;
      const auto hp = read_ints(in, H + 1);
      const int total = hp[H] > 0 ? hp[H] : 0;
      const auto offs = read_ints(in, total);
      const fibatt_table_desc d{B, H, N, D, dt, cls, hp.data(), total ? offs.data() : nullptr,
                                total ? offs.data() : nullptr};
      std::cout << fibatt_bwd_table_workspace_floats(&d) << "\n";
    } else if (op == "layouts") {
      int32_t bwd, B, H, N, D, dt;
      in >> bwd >> B >> H >> N >> D >> dt;
      fibatt_layouts ls{};
      fibatt_layout* all[8] = {&ls.q, &ls.k, &ls.v, &ls.o, &ls.dout, &ls.dq, &ls.dk, &ls.dv};
      for (fibatt_layout* l : all) {
        long long sb, sh, sn;
        in >> sb >> sh >> sn;
        *l = fibatt_layout{sb, sh, sn};
      }
      const int32_t one = 1;
      const int32_t wN = N;
      std::vector<int32_t> a(H > 0 ? H : 1, 1), b(H > 0 ? H : 1, 2), w(H > 0 ? H : 1, wN);
      (void)one;
      const fibatt_desc d{B, H, N, D, dt, a.data(), b.data(), w.data()};
      fibatt::Problem p;
      int rc = fibatt::host::check_desc(&d, &p);
      if (rc == FIBATT_OK) rc = fibatt::host::check_layouts(&ls, bwd != 0, &p);
      std::cout << rc << " " << (rc == FIBATT_OK ? static_cast<int>(p.strided) : -1) << "\n";
    } else if (!op.empty()) {
      std::cout << "?\n";
    }
  }
  return 0;
}
