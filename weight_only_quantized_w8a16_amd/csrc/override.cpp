// override.cpp -- the one dispatch override of libqgemm (qg_set_override in
// include/qgemm.h): tests and tuning force the choices the host dispatch
// otherwise makes from a problem's sizes (decode or prefill path, prefill
// tile and split-K slices, MoE tile, W8A8 tile and slices).  The environment
// variable QGEMM_OVERRIDE gives the initial setting and is read once, on the
// first dispatch; qg_set_override replaces the setting afterwards.  Nothing
// else in the library reads the environment.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qgemm.h"
#include "qg_launch.hpp"

namespace qg {

namespace {

std::mutex g_mu;
Override g_ov;
bool g_init = false;

bool parse_int(const std::string &v, int lo, int hi, int &out) {
  if (v.empty()) return false;
  char *end = nullptr;
  const long x = std::strtol(v.c_str(), &end, 10);
  if (*end != '\0' || x < lo || x > hi) return false;
  out = static_cast<int>(x);
  return true;
}

// Parses `spec` into `o` (starting from the automatic choices); false on an
// unknown key or value.
bool parse(const char *spec, Override &o) {
  o = Override{};
  if (!spec) return true;
  const std::string s(spec);
  size_t pos = 0;
  while (pos <= s.size()) {
    size_t end = s.find(',', pos);
    if (end == std::string::npos) end = s.size();
    const std::string item = s.substr(pos, end - pos);
    pos = end + 1;
    if (item.empty()) continue;
    const size_t eq = item.find('=');
    if (eq == std::string::npos) return false;
    const std::string k = item.substr(0, eq), v = item.substr(eq + 1);
    if (k == "path") {
      if (v == "auto") o.path = kPathAuto;
      else if (v == "decode") o.path = kPathDecode;
      else if (v == "prefill") o.path = kPathPrefill;
      else return false;
    } else if (k == "prefill_tile") {
      static const char *names[] = {"X", "D8", "D8N", "D64", "D128", "L", "M", "S", "P256", "P128", "P64",
                                    "W256", "W256N", "W128", "W64", "WX", "DX"};
      int t = -1;
      for (int i = 0; i < static_cast<int>(sizeof(names) / sizeof(names[0])); ++i)
        if (v == names[i]) t = i;
      if (t < 0 && v != "auto") return false;
      o.prefill_tile = t;
    } else if (k == "splitk") {
      if (!parse_int(v, 1, 1024, o.splitk)) return false;
    } else if (k == "moe_tile") {
      if (v == "auto") o.moe_small_tile = false;
      else if (v == "S") o.moe_small_tile = true;
      else return false;
    } else if (k == "w8a8_tile") {
      static const char *names[] = {"T256", "T256N", "T128", "T64"};
      int t = -1;
      for (int i = 0; i < 4; ++i)
        if (v == names[i]) t = i;
      if (t < 0 && v != "auto") return false;
      o.w8a8_tile = t;
    } else if (k == "w8a8_split") {
      if (!parse_int(v, 1, 1024, o.w8a8_split)) return false;
    } else {
      return false;
    }
    if (end == s.size()) break;
  }
  return true;
}

}  // namespace

Override dispatch_override() {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_init) {
    Override o;
    if (parse(std::getenv("QGEMM_OVERRIDE"), o)) g_ov = o;
    g_init = true;
  }
  return g_ov;
}

}  // namespace qg

extern "C" qg_status qg_set_override(const char *spec) {
  qg::Override o;
  if (!qg::parse(spec, o)) return QG_ERR_MODE;
  std::lock_guard<std::mutex> lk(qg::g_mu);
  qg::g_ov = o;
  qg::g_init = true;
  return QG_OK;
}
