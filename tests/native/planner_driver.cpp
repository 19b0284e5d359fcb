// CPU test driver for the host planner, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_planner_sanitized.py (plain g++,
// no GPU code).  Reads one request per line on stdin and answers on stdout:
//
//   plan Tq Tk bm bn transpose R  qs qe ks ke type  (R times)
//     -> "ok N" and N lines "tile other r kind", or "error <message>"
//   block Tq Tk block_q block_k width n_qblocks  num[n_qblocks]  idx[n_qblocks*width]
//     -> "ok N" and N lines "qs qe ks ke", or "error <message>"
//   disjoint Tq Tk R  qs qe ks ke type  (R times)
//     -> "ok" or "overlap <message>" (slices must first pass validation)
//
// Every number is read as a 64-bit integer and passed on as int32 where the
// planner takes int32, so out-of-range values reach the planner's checks.
#include <cstdint>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "planner.hpp"

namespace {

bool read_slices(std::istream& in, int64_t R, std::vector<int32_t>* qr, std::vector<int32_t>* kr,
                 std::vector<int32_t>* ty) {
  if (R < 0 || R > (1 << 20)) return false;
  qr->resize(2 * R);
  kr->resize(2 * R);
  ty->resize(R);
  for (int64_t r = 0; r < R; ++r) {
    int64_t a, b, c, d, t;
    if (!(in >> a >> b >> c >> d >> t)) return false;
    (*qr)[2 * r] = (int32_t)a;
    (*qr)[2 * r + 1] = (int32_t)b;
    (*kr)[2 * r] = (int32_t)c;
    (*kr)[2 * r + 1] = (int32_t)d;
    (*ty)[r] = (int32_t)t;
  }
  return true;
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    if (cmd == "plan" || cmd == "disjoint") {
      int64_t Tq, Tk, bm = 1, bn = 1, tr = 0, R;
      if (!(in >> Tq >> Tk)) return 2;
      if (cmd == "plan" && !(in >> bm >> bn >> tr)) return 2;
      if (!(in >> R)) return 2;
      std::vector<int32_t> qr, kr, ty;
      if (!read_slices(in, R, &qr, &kr, &ty)) return 2;
      std::vector<ffa::Slice> slices;
      std::string m = ffa::validate_slices(Tq, Tk, qr.data(), kr.data(), ty.data(), (int)R, &slices);
      if (!m.empty()) {
        std::cout << "error " << m << "\n";
        continue;
      }
      if (cmd == "disjoint") {
        m = ffa::check_disjoint(slices);
        std::cout << (m.empty() ? std::string("ok") : "overlap " + m) << "\n";
        continue;
      }
      if (bm <= 0 || bn <= 0) {
        std::cout << "error tile sizes must be positive\n";
        continue;
      }
      ffa::Plan plan;
      ffa::build_plan(slices, Tq, Tk, (int)bm, (int)bn, tr != 0, &plan);
      std::cout << "ok " << plan.entries.size() << "\n";
      for (int64_t t = 0; t < plan.n_tiles; ++t)
        for (int64_t e = plan.row_ptr[t]; e < plan.row_ptr[t + 1]; ++e) {
          const ffa::PlanEntry& pe = plan.entries[e];
          std::cout << t << " " << pe.other << " " << slices[pe.slice].r << " " << pe.kind << "\n";
        }
    } else if (cmd == "block") {
      int64_t Tq, Tk, bq, bk, width, nqb;
      if (!(in >> Tq >> Tk >> bq >> bk >> width >> nqb)) return 2;
      if (nqb < 0 || width < 0 || nqb > (1 << 16) || width > (1 << 16)) return 2;
      // the planner reads one count per query block of the token axis
      if (bq > 0 && Tq >= 0 && nqb != (Tq + bq - 1) / bq) return 2;
      std::vector<int32_t> num(nqb), idx(nqb * width);
      for (auto& x : num) {
        int64_t v;
        if (!(in >> v)) return 2;
        x = (int32_t)v;
      }
      for (auto& x : idx) {
        int64_t v;
        if (!(in >> v)) return 2;
        x = (int32_t)v;
      }
      std::vector<ffa::RangePair> out;
      std::string m = ffa::block_slices(Tq, Tk, (int)bq, (int)bk, num.data(), idx.data(), (int)width, &out);
      if (!m.empty()) {
        std::cout << "error " << m << "\n";
        continue;
      }
      std::cout << "ok " << out.size() << "\n";
      for (const auto& p : out) std::cout << p.qs << " " << p.qe << " " << p.ks << " " << p.ke << "\n";
    } else {
      return 2;
    }
  }
  return 0;
}
