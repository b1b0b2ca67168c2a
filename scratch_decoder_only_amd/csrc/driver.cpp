// Multi-step training around train_step (the learning-rate schedule and
// checkpoint files) and the host side of generation (next-token choice).
//
// Schedule (LucilleAI page, usage of the SFT trainer: a cosine scheduler with
// warm-up steps and a minimum learning rate): linear warm-up to lr_max, then a
// half cosine down to lr_min at the last step.
//
// Checkpoints (LucilleAI page: save every N steps, resume with --init-from;
// Smallem page, "Les règles du jeu": weight files carry a JSON header): one
// file in the safetensors layout, an 8-byte little-endian header length, a
// JSON header, then raw little-endian fp32 tensors. It holds the parameters
// and both Adam moments, tensor by tensor in the parameter-table order, and
// the step and model dimensions as string metadata. Written to path + ".tmp"
// and renamed, so a crash never leaves a torn file under the final name.
#include <hip/hip_runtime.h>

#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/lmstep.h"
#include "host.h"
#include "kernels.h"

using lm::set_error;

extern "C" float lm_lr_schedule(int32_t step, int32_t warmup_steps, int32_t total_steps, float lr_max,
                                float lr_min) {
  const double s = step < 1 ? 1.0 : (double)step;
  if (warmup_steps > 0 && s <= warmup_steps) return (float)(lr_max * s / warmup_steps);
  if (total_steps <= warmup_steps || total_steps <= 0) return lr_max;  // no decay phase
  if (s >= total_steps) return lr_min;
  const double p = (s - warmup_steps) / (double)(total_steps - warmup_steps);
  return (float)(lr_min + 0.5 * ((double)lr_max - lr_min) * (1.0 + std::cos(M_PI * p)));
}

namespace {

const char* kFormat = "lmstep-checkpoint";

struct Table {
  std::vector<lm_tensor_info> t;
  int64_t P = 0;
};

lm_status read_table(const lm_model* m, Table& tb) {
  int32_t n = 0;
  lm_status st = model_param_table(m, nullptr, &n, &tb.P);
  if (st != LM_OK) return st;
  tb.t.resize(n);
  return model_param_table(m, tb.t.data(), &n, &tb.P);
}

// The buffers a checkpoint holds, with their tensor-name prefixes.
struct Section {
  lm_buf buf;
  const char* prefix;
};
const Section kSections[3] = {{LM_PARAMS, "param."}, {LM_ADAM_M, "adam_m."}, {LM_ADAM_V, "adam_v."}};

std::map<std::string, std::string> config_meta(const lm_config& c, int32_t step) {
  char eps[32];
  std::snprintf(eps, sizeof(eps), "%.9g", (double)c.ln_eps);
  return {{"format", kFormat},
          {"version", "1"},
          {"step", std::to_string(step)},
          {"vocab", std::to_string(c.vocab)},
          {"d_model", std::to_string(c.d_model)},
          {"n_heads", std::to_string(c.n_heads)},
          {"d_mlp", std::to_string(c.d_mlp)},
          {"n_layers", std::to_string(c.n_layers)},
          {"max_seq", std::to_string(c.max_seq)},
          {"precision", std::to_string(c.precision)},
          {"ln_eps", eps},
          {"untied_head", std::to_string(c.untied_head)}};
}

std::string shape_json(const lm_tensor_info& t) {
  return t.cols == 1 ? "[" + std::to_string(t.rows) + "]"
                     : "[" + std::to_string(t.rows) + "," + std::to_string(t.cols) + "]";
}

// ------------------------------------------------------ minimal JSON reader
// Enough for the header: objects, arrays, strings, integers (and the other
// literals, which are skipped).
struct JVal {
  enum Kind { NUL, NUM, STR, ARR, OBJ, BOOL } kind = NUL;
  double num = 0;
  std::string str;
  std::vector<JVal> arr;
  std::map<std::string, JVal> obj;
};

struct JParser {
  const char* p;
  const char* end;
  bool ok = true;
  void ws() {
    while (p < end && std::isspace((unsigned char)*p)) ++p;
  }
  bool eat(char c) {
    ws();
    if (p < end && *p == c) {
      ++p;
      return true;
    }
    return false;
  }
  std::string string() {
    std::string out;
    if (!eat('"')) {
      ok = false;
      return out;
    }
    while (p < end && *p != '"') {
      char c = *p++;
      if (c == '\\' && p < end) {
        char e = *p++;
        switch (e) {
          case 'n': out += '\n'; break;
          case 't': out += '\t'; break;
          case 'r': out += '\r'; break;
          case 'b': out += '\b'; break;
          case 'f': out += '\f'; break;
          case 'u': p = p + 4 <= end ? p + 4 : end; out += '?'; break;
          default: out += e;
        }
      } else {
        out += c;
      }
    }
    if (p >= end) ok = false;
    else ++p;
    return out;
  }
  JVal value(int depth = 0) {
    JVal v;
    ws();
    if (p >= end || depth > 16) {
      ok = false;
      return v;
    }
    if (*p == '{') {
      ++p;
      v.kind = JVal::OBJ;
      if (eat('}')) return v;
      do {
        std::string k = string();
        if (!ok || !eat(':')) {
          ok = false;
          return v;
        }
        v.obj[k] = value(depth + 1);
      } while (ok && eat(','));
      if (!eat('}')) ok = false;
    } else if (*p == '[') {
      ++p;
      v.kind = JVal::ARR;
      if (eat(']')) return v;
      do v.arr.push_back(value(depth + 1));
      while (ok && eat(','));
      if (!eat(']')) ok = false;
    } else if (*p == '"') {
      v.kind = JVal::STR;
      v.str = string();
    } else if (*p == '-' || std::isdigit((unsigned char)*p)) {
      char* q = nullptr;
      v.kind = JVal::NUM;
      v.num = std::strtod(p, &q);
      if (q == p) ok = false;
      p = q;
    } else {
      const char* words[3] = {"true", "false", "null"};
      for (const char* w : words) {
        size_t n = std::strlen(w);
        if ((size_t)(end - p) >= n && std::strncmp(p, w, n) == 0) {
          p += n;
          v.kind = w[0] == 'n' ? JVal::NUL : JVal::BOOL;
          return v;
        }
      }
      ok = false;
    }
    return v;
  }
};

struct File {
  std::FILE* f = nullptr;
  ~File() {
    if (f) std::fclose(f);
  }
};

}  // namespace

extern "C" {

lm_status model_save(const lm_model* m, const char* path, int32_t step, void* stream) {
  if (!m || !path) return set_error(LM_ERR_ARG, "model or path is NULL");
  lm_config cfg;
  lm_status st = model_config(m, &cfg);
  if (st != LM_OK) return st;
  Table tb;
  if ((st = read_table(m, tb)) != LM_OK) return st;

  // header: every tensor of every section, data offsets back to back
  std::map<std::string, std::string> meta = config_meta(cfg, step);
  if (cfg.precision == 2) {
    // the dynamic loss scale is part of an fp16 run's state
    lm_loss_scaler ls;
    if ((st = model_get_loss_scaler(m, &ls, stream)) != LM_OK) return st;
    char v[32];
    std::snprintf(v, sizeof(v), "%.9g", (double)ls.scale);
    meta["loss_scale"] = v;
    std::snprintf(v, sizeof(v), "%.9g", (double)ls.growth);
    meta["loss_scale_growth"] = v;
    std::snprintf(v, sizeof(v), "%.9g", (double)ls.backoff);
    meta["loss_scale_backoff"] = v;
    meta["loss_scale_interval"] = std::to_string(ls.interval);
    meta["loss_scale_good_steps"] = std::to_string(ls.good_steps);
  }
  std::string h = "{\"__metadata__\":{";
  bool first = true;
  for (const auto& kv : meta) {
    h += (first ? "\"" : ",\"") + kv.first + "\":\"" + kv.second + "\"";
    first = false;
  }
  h += "}";
  uint64_t off = 0;
  for (const Section& sec : kSections)
    for (const auto& t : tb.t) {
      const uint64_t n = (uint64_t)t.rows * t.cols * 4;
      h += ",\"" + std::string(sec.prefix) + t.name + "\":{\"dtype\":\"F32\",\"shape\":" + shape_json(t) +
           ",\"data_offsets\":[" + std::to_string(off) + "," + std::to_string(off + n) + "]}";
      off += n;
    }
  h += "}";
  while (h.size() % 8) h += ' ';

  const std::string tmp = std::string(path) + ".tmp";
  File out;
  out.f = std::fopen(tmp.c_str(), "wb");
  if (!out.f) return set_error(LM_ERR_ARG, "cannot open " + tmp + " for writing");
  unsigned char len[8];
  for (int i = 0; i < 8; ++i) len[i] = (unsigned char)(((uint64_t)h.size() >> (8 * i)) & 0xff);
  bool good = std::fwrite(len, 1, 8, out.f) == 8 && std::fwrite(h.data(), 1, h.size(), out.f) == h.size();
  std::unique_ptr<float[]> host(new float[tb.P]);
  for (const Section& sec : kSections) {
    if (!good) break;
    if ((st = model_get(m, sec.buf, host.get(), 0, stream)) != LM_OK) return st;
    for (const auto& t : tb.t) {
      const size_t n = (size_t)t.rows * t.cols;
      if (std::fwrite(host.get() + t.offset, 4, n, out.f) != n) {
        good = false;
        break;
      }
    }
  }
  good = good && std::fflush(out.f) == 0;
  good = std::fclose(out.f) == 0 && good;
  out.f = nullptr;
  if (!good) {
    std::remove(tmp.c_str());
    return set_error(LM_ERR_ARG, "writing " + tmp + " failed");
  }
  if (std::rename(tmp.c_str(), path) != 0) {
    std::remove(tmp.c_str());
    return set_error(LM_ERR_ARG, std::string("cannot rename the checkpoint to ") + path);
  }
  return LM_OK;
}

lm_status model_load(lm_model* m, const char* path, int32_t* step, void* stream) {
  if (!m || !path) return set_error(LM_ERR_ARG, "model or path is NULL");
  lm_config cfg;
  lm_status st = model_config(m, &cfg);
  if (st != LM_OK) return st;
  Table tb;
  if ((st = read_table(m, tb)) != LM_OK) return st;

  File in;
  in.f = std::fopen(path, "rb");
  if (!in.f) return set_error(LM_ERR_ARG, std::string("cannot open ") + path);
  unsigned char len[8];
  if (std::fread(len, 1, 8, in.f) != 8) return set_error(LM_ERR_ARG, "checkpoint too short");
  uint64_t hn = 0;
  for (int i = 0; i < 8; ++i) hn |= (uint64_t)len[i] << (8 * i);
  if (hn == 0 || hn > (64u << 20)) return set_error(LM_ERR_ARG, "checkpoint header length is not plausible");
  std::string h(hn, '\0');
  if (std::fread(&h[0], 1, hn, in.f) != hn) return set_error(LM_ERR_ARG, "checkpoint header is truncated");
  JParser jp{h.data(), h.data() + h.size()};
  JVal root = jp.value();
  if (!jp.ok || root.kind != JVal::OBJ) return set_error(LM_ERR_ARG, "checkpoint header is not a JSON object");

  // metadata: format and every model dimension must match this model
  auto meta_it = root.obj.find("__metadata__");
  if (meta_it == root.obj.end() || meta_it->second.kind != JVal::OBJ)
    return set_error(LM_ERR_ARG, "checkpoint has no metadata");
  const auto& meta = meta_it->second.obj;
  auto meta_str = [&](const char* k) -> std::string {
    auto it = meta.find(k);
    return it != meta.end() && it->second.kind == JVal::STR ? it->second.str : std::string("<missing>");
  };
  if (meta_str("format") != kFormat) return set_error(LM_ERR_ARG, "not an lmstep checkpoint");
  for (const auto& kv : config_meta(cfg, 0)) {
    if (kv.first == "step" || kv.first == "format" || kv.first == "version") continue;
    // files written before the separate head existed hold the tied model
    if (kv.first == "untied_head" && meta_str("untied_head") == "<missing>" && kv.second == "0") continue;
    if (meta_str(kv.first.c_str()) != kv.second)
      return set_error(LM_ERR_SHAPE, "checkpoint " + kv.first + " = " + meta_str(kv.first.c_str()) +
                                         " does not match the model's " + kv.second);
  }
  const std::string step_s = meta_str("step");
  char* endp = nullptr;
  const long saved_step = std::strtol(step_s.c_str(), &endp, 10);
  if (endp == step_s.c_str()) return set_error(LM_ERR_ARG, "checkpoint step is not a number");

  // every tensor: F32, the model's shape, offsets inside the data section
  const long data_start = 8 + (long)hn;
  std::fseek(in.f, 0, SEEK_END);
  const long file_size = std::ftell(in.f);
  std::unique_ptr<float[]> host(new float[tb.P]);
  for (const Section& sec : kSections) {
    std::memset(host.get(), 0, (size_t)tb.P * 4);
    for (const auto& t : tb.t) {
      const std::string name = std::string(sec.prefix) + t.name;
      auto it = root.obj.find(name);
      if (it == root.obj.end() || it->second.kind != JVal::OBJ)
        return set_error(LM_ERR_ARG, "checkpoint lacks " + name);
      const auto& e = it->second.obj;
      auto dt = e.find("dtype"), sh = e.find("shape"), of = e.find("data_offsets");
      if (dt == e.end() || dt->second.str != "F32") return set_error(LM_ERR_ARG, name + " is not F32");
      std::vector<int64_t> want = t.cols == 1 ? std::vector<int64_t>{t.rows} : std::vector<int64_t>{t.rows, t.cols};
      bool shape_ok = sh != e.end() && sh->second.kind == JVal::ARR && sh->second.arr.size() == want.size();
      for (size_t i = 0; shape_ok && i < want.size(); ++i) shape_ok = (int64_t)sh->second.arr[i].num == want[i];
      if (!shape_ok) return set_error(LM_ERR_SHAPE, name + " has another shape in the checkpoint");
      if (of == e.end() || of->second.kind != JVal::ARR || of->second.arr.size() != 2)
        return set_error(LM_ERR_ARG, name + " has no data offsets");
      const long b = (long)of->second.arr[0].num, en = (long)of->second.arr[1].num;
      const size_t n = (size_t)t.rows * t.cols;
      if (b < 0 || en - b != (long)(n * 4) || data_start + en > file_size)
        return set_error(LM_ERR_ARG, name + " has inconsistent data offsets");
      if (std::fseek(in.f, data_start + b, SEEK_SET) != 0 || std::fread(host.get() + t.offset, 4, n, in.f) != n)
        return set_error(LM_ERR_ARG, "reading " + name + " failed");
    }
    if ((st = model_set(m, sec.buf, host.get(), 0, stream)) != LM_OK) return st;
  }
  if (cfg.precision == 2 && meta_str("loss_scale") != "<missing>") {
    lm_loss_scaler ls;
    ls.scale = std::strtof(meta_str("loss_scale").c_str(), nullptr);
    ls.growth = std::strtof(meta_str("loss_scale_growth").c_str(), nullptr);
    ls.backoff = std::strtof(meta_str("loss_scale_backoff").c_str(), nullptr);
    ls.interval = (int32_t)std::strtol(meta_str("loss_scale_interval").c_str(), nullptr, 10);
    ls.good_steps = (int32_t)std::strtol(meta_str("loss_scale_good_steps").c_str(), nullptr, 10);
    if ((st = model_set_loss_scaler(m, &ls, stream)) != LM_OK) return st;
  }
  if (step) *step = (int32_t)saved_step;
  return LM_OK;
}

lm_status sample_tokens(const float* d_logits, int32_t rows, int32_t vocab, int64_t ld, float temperature,
                        int32_t top_k, const float* d_uniforms, int32_t* d_out, void* stream) {
  if (!d_logits || !d_out) return set_error(LM_ERR_ARG, "logits or out is NULL");
  if (rows < 0 || vocab < 1 || ld < vocab) return set_error(LM_ERR_SHAPE, "need rows >= 0, vocab >= 1, ld >= vocab");
  if (temperature > 0.f && !d_uniforms) return set_error(LM_ERR_ARG, "sampling needs one uniform per row");
  if (rows == 0) return LM_OK;
  lm::launch_sample(d_logits, rows, vocab, (long)ld, temperature, top_k, d_uniforms, d_out,
                    reinterpret_cast<hipStream_t>(stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(LM_ERR_HIP, std::string("sample_tokens: ") + hipGetErrorString(e));
  return LM_OK;
}

}  // extern "C"
