"""MI355X-native absorbed MLA decode library (binding loaded lazily)."""
