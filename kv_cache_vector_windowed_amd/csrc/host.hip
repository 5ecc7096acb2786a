// Library-wide host entry points: status text, version, retrieval-set size and the
// optional per-kernel event timing.
#include <cstdio>
#include <string>
#include <vector>

#include "common.hpp"

namespace a2ats {
namespace {

struct ProfRecord {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};

bool g_prof_on = false;
std::vector<ProfRecord> g_prof;

}  // namespace

void profile_begin(const char* name, hipStream_t s, int* slot) {
  *slot = -1;
  if (!g_prof_on) return;
  ProfRecord r{name, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess) return;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return;
  }
  (void)hipEventRecord(r.start, s);
  g_prof.push_back(r);
  *slot = static_cast<int>(g_prof.size()) - 1;
}

void profile_end(int slot, hipStream_t s) {
  if (slot < 0 || slot >= static_cast<int>(g_prof.size())) return;
  (void)hipEventRecord(g_prof[slot].stop, s);
}

}  // namespace a2ats

extern "C" {

const char* a2ats_strerror(int status) {
  switch (status) {
    case A2ATS_OK: return "ok";
    case A2ATS_EINVAL: return "invalid argument";
    case A2ATS_EDTYPE: return "unsupported dtype";
    case A2ATS_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case A2ATS_ENOTSPD: return "matrix is not positive definite";
    case A2ATS_EHIP: return "HIP runtime error";
    case A2ATS_ESCRATCH: return "larger than the fixed scratch of an allocation-free call";
    default: return "unknown status";
  }
}

int a2ats_version(void) { return A2ATS_VERSION; }

int64_t a2ats_retrieval_count(int64_t n, double fraction) {
  if (n < 0 || !(fraction >= 0.0 && fraction <= 1.0)) return -1;
  return static_cast<int64_t>(std::ceil(fraction * static_cast<double>(n)));
}

int a2ats_profile_enable(int on) {
  a2ats::g_prof_on = (on != 0);
  return A2ATS_OK;
}

int a2ats_profile_reset(void) {
  for (auto& r : a2ats::g_prof) {
    (void)hipEventSynchronize(r.stop);
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  a2ats::g_prof.clear();
  return A2ATS_OK;
}

int64_t a2ats_profile_read(char* buf, size_t len) {
  std::vector<std::string> names;
  std::vector<long> counts;
  std::vector<double> totals;
  for (auto& r : a2ats::g_prof) {
    if (hipEventSynchronize(r.stop) != hipSuccess) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) continue;
    size_t k = 0;
    for (; k < names.size(); ++k)
      if (names[k] == r.name) break;
    if (k == names.size()) {
      names.emplace_back(r.name);
      counts.push_back(0);
      totals.push_back(0.0);
    }
    counts[k] += 1;
    totals[k] += ms;
  }
  std::string out;
  char line[256];
  for (size_t k = 0; k < names.size(); ++k) {
    snprintf(line, sizeof line, "%s\t%ld\t%.6f\n", names[k].c_str(), counts[k], totals[k]);
    out += line;
  }
  if (buf && len > 0) {
    size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = '\0';
  }
  return static_cast<int64_t>(out.size() + 1);
}

}  // extern "C"
